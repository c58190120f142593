// fa2_fwd_roles.hpp -- exact attention forward with the two waves of a SIMD
// in different roles: one computes scores and the online softmax, the other
// accumulates P.V one key tile behind.
//
// The work partition is the one of the "FlashAttention v2 better parallelism
// + work partitioning" diagram (grid over query blocks and heads, query rows
// split across waves, K/V tiles shared through LDS); the split of one query
// slice's work between a softmax role and a matrix-multiply role follows the
// role split of the "FlashAttention v4 Blackwell pipeline co-design"
// diagram.  Per workgroup 8 waves, two per SIMD, own 128 queries: wave w and
// wave w+4 (same SIMD) form pair w, which owns queries [q_wg + 32w, +32).
//   * the S wave (w < 4) keeps the pair's Q rows in VGPRs, computes
//     S^T = K Q^T of key tile j and the online softmax (running max and sum,
//     lazy rescale as in fa2_fwd_kernel), and stores the packed 16-bit P^T
//     and the per-query rescale factor alpha in LDS;
//   * the PV wave (w >= 4) keeps O^T in registers; in the next iteration it
//     reads alpha and P^T of tile j (the same lane layout as the S wave's
//     registers: lane % 32 is the query), rescales O^T when some row moved
//     and accumulates O^T += V^T P^T with V^T through the transpose read.
// So while one wave of a SIMD runs its softmax the other issues MFMAs.  K and
// V tiles are copied straight from memory into two 3-stage LDS rings by
// inline-assembly copies, two iterations ahead; one barrier per iteration
// publishes the next K and V tiles and the P slots.  At the end the S wave
// writes LSE and hands the row sums to the PV wave, which writes O = O^T / l.
#pragma once

#include "fa2_fwd_kernel.hpp"

namespace fa2 {

template <bool BF16, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fa2_fwd_roles_kernel(Args a) {
  using E = Elem<BF16>;
  constexpr int BR = 128;                   // queries per workgroup
  constexpr int BC = 64;                    // keys per tile
  constexpr int KB = BC / 32;
  constexpr int DK = D / 16, DB = D / 32, KROW = D * 2;
  constexpr int TSZ = BC * KROW;            // bytes of one K (or V) tile
  constexpr int NSK = 3, NSV = 3;           // ring stages
  constexpr int PSLOT = 4 * 64 * 16;        // packed P^T of one pair and tile: 4 x 16 bytes per lane
  constexpr int KBASE = 0, VBASE = NSK * TSZ, PBASE = VBASE + NSV * TSZ;
  constexpr int ABASE = PBASE + 4 * 2 * PSLOT;       // alpha: 4 pairs x 2 slots x 32 floats
  constexpr int LBASE = ABASE + 4 * 2 * 32 * 4;      // row sums: 4 pairs x 32 floats
  constexpr int SMEM = LBASE + 4 * 32 * 4;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int pair = wv & 3;
  const bool pv_role = wv >= 4;

  int bh, qblk;
  {
    const int i = blockIdx.x;
    const int total = a.nqb * a.BH;
    if constexpr (!CAUSAL) {
      const int logical = (total % 8 == 0) ? (i % 8) * (total / 8) + i / 8 : i;
      bh = logical / a.nqb;
      qblk = logical % a.nqb;
    } else {
      bh = i % a.BH;
      qblk = a.nqb - 1 - i / a.BH;
    }
  }
  const int N = a.N;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.q + head_off), 0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.k + head_off), 0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.v + head_off), 0, head_bytes, kBufferWord3);

  const int q_wg = qblk * BR;
  const int q_w = q_wg + 32 * pair;         // first query of the pair
  const int q = q_w + lr;                   // this lane's query

  int nt = (N + BC - 1) / BC;
  if constexpr (CAUSAL) {
    const int last_row = min(q_wg + BR, N) - 1;
    nt = min(nt, last_row / BC + 1);
  }
  auto tile_skip = [&](int key0) { return CAUSAL && key0 > q_w + 31; };
  auto tile_masked = [&](int key0) { return (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q_w); };

  // ---- S wave state: Q fragments (B operands), running max and sum --------
  u32x4 qf[DK];
  const bool c_neg = a.c < 0.f;
  const float c = c_neg ? -a.c : a.c;
  if (!pv_role) {
#pragma unroll
    for (int dk = 0; dk < DK; ++dk)
      qf[dk] = __builtin_amdgcn_raw_buffer_load_b128(qr, (uint32_t)(q * KROW + (2 * dk + lh) * 16), 0, 0);
  } else {
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) qf[dk] = u32x4{};
  }
  float m_run = -INFINITY, l_run = 0.f;
  // ---- PV wave state: O^T accumulator ---------------------------------------
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // ---- copies: K and V rings, 1 KiB per instruction, 2 (d = 128) or 1 per wave and tensor
  constexpr int NI = TSZ / 1024;
  constexpr int IPW = NI / 8;
  static_assert(NI % 8 == 0 && IPW >= 1, "tile copies must split evenly over the waves");
  uint32_t dsrc[IPW];
#pragma unroll
  for (int k = 0; k < IPW; ++k) {
    const int b = (wv * IPW + k) * 1024 + 16 * lane;
    const int row = b / KROW, phys = (b % KROW) / 16;
    dsrc[k] = (uint32_t)(row * KROW + 16 * (phys ^ chunk_swizzle<D>(row)));
  }
  auto copy_k = [&](int j) {
#pragma unroll
    for (int k = 0; k < IPW; ++k)
      lds_dma16_asm(kr, smem + KBASE + (j % NSK) * TSZ + (wv * IPW + k) * 1024, dsrc[k], j * BC * KROW);
  };
  auto copy_v = [&](int j) {
#pragma unroll
    for (int k = 0; k < IPW; ++k)
      lds_dma16_asm(vr, smem + VBASE + (j % NSV) * TSZ + (wv * IPW + k) * 1024, dsrc[k], j * BC * KROW);
  };

  // fragment addresses (see chunk_swizzle): K row 32*kb + lr, chunk 2*dk + lh;
  // V^T through the transpose read (as in fa2_fwd_kernel)
  const int kfb = lr * KROW + 16 * (lh ^ chunk_swizzle<D>(lr));
  const int vgq = lane >> 4, ve = (lane >> 2) & 3, vc = lane & 3;
  const int vfb = (4 * (vgq >> 1) + ve) * KROW + 8 * (vc & 1) + (D == 128 ? 64 * ve : 64 * (ve >> 1)) +
                  16 * ((2 * (vgq & 1) | (vc >> 1)) ^ (vgq >> 1));

  uint8_t* const pslot = smem + PBASE + pair * 2 * PSLOT + 16 * lane;   // + parity * PSLOT + idx * 1024
  float* const aslot = (float*)(smem + ABASE) + pair * 2 * 32;          // + parity * 32 + query
  float* const lslot = (float*)(smem + LBASE) + pair * 32;

  // S wave, tile j: scores, online softmax, P^T and alpha to LDS slot j % 2
  auto s_tile = [&](int j) {
    const int key0 = j * BC;
    const uint8_t* kt = smem + KBASE + (j % NSK) * TSZ;
    f32x16 sv[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sv[kb] = f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; ++dk)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        sv[kb] = E::mfma(*(const u32x4*)(kt + (kfb ^ (32 * dk)) + 32 * kb * KROW), qf[dk], sv[kb]);
    float cc = c, m_tile;
    if (tile_masked(key0)) {
      float e0 = -INFINITY, e1 = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * lh + (r & 3);
          const bool vis = key < N && (!CAUSAL || key <= q);
          const float t = vis ? sv[kb][r] * c : -INFINITY;
          sv[kb][r] = t;
          if (r & 1) e1 = fmaxf(e1, t); else e0 = fmaxf(e0, t);
        }
      m_tile = max_halves(fmaxf(e0, e1));
      cc = 1.f;
    } else {
      float e0 = sv[0][0], e1 = sv[0][1];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          e0 = fmaxf(e0, fmaxf(sv[kb][r], sv[kb][r + 1]));
          e1 = fmaxf(e1, fmaxf(sv[kb][r + 2], sv[kb][r + 3]));
        }
      m_tile = max_halves(fmaxf(e0, e1)) * c;
    }
    const float m_old = m_run;
    const float m_new = (m_tile > m_old + kLazyRescale) ? m_tile : m_old;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_old - m_use);
    m_run = m_new;
    float rs0 = 0.f, rs1 = 0.f;
    uint8_t* ps = pslot + (j & 1) * PSLOT;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float p[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kb][8 * st + t], cc, -m_use));
          if (t & 1) rs1 += p[t]; else rs0 += p[t];
        }
        u32x4 pw;
#pragma unroll
        for (int t = 0; t < 4; ++t) pw[t] = E::pack(p[2 * t], p[2 * t + 1]);
        *(u32x4*)(ps + (2 * kb + st) * 1024) = pw;
      }
    }
    l_run = l_run * alpha + (rs0 + rs1);
    if (lh == 0) aslot[(j & 1) * 32 + lr] = alpha;
  };

  // PV wave, tile j: rescale O^T by alpha when some row moved, O^T += V^T P^T
  auto pv_tile = [&](int j) {
    const uint8_t* vt = smem + VBASE + (j % NSV) * TSZ;
    const uint8_t* ps = pslot + (j & 1) * PSLOT;
    const float alpha = aslot[(j & 1) * 32 + lr];
    u32x4 pf[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) pf[kb][st] = *(const u32x4*)(ps + (2 * kb + st) * 1024);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint8_t* vp = vt + (32 * kb + 16 * st) * KROW;
          const u32x2 lo = lds_read_tr16(vp + (vfb ^ (64 * db)));
          const u32x2 hi = lds_read_tr16(vp + 8 * KROW + (vfb ^ (64 * db) ^ 32));
          acc[db] = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kb][st], acc[db]);
        }
  };

  // ---- prologue: K_0, K_1, V_0 in flight; the negative-scale fold ---------
  if (!pv_role && c_neg) {
    const u32x4 sign = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) qf[dk] ^= sign;
  }
  copy_k(0);
  if (nt > 1) copy_k(1);
  copy_v(0);
  // this wave's copies of K_0 have landed once only K_1's and V_0's remain
  if (nt > 1) FA2_WAIT_VMCNT(2 * IPW); else FA2_WAIT_VMCNT(IPW);
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) asm volatile("" ::"v"(qf[dk]));
  __syncthreads();

  // ---- iteration j: S wave on tile j, PV wave on tile j-1 -------------------
  for (int j = 0; j <= nt; ++j) {
    // the barrier that ended iteration j-1 freed K stage (j+2)%3 (last read in
    // j-1... tile j-1) and V stage (j+1)%3 (tile j-2, read in j-1)
    const bool ck = j + 2 < nt, cv = j + 1 < nt;
    if (ck) copy_k(j + 2);
    if (cv) copy_v(j + 1);
    if (!pv_role) {
      if (j < nt && !tile_skip(j * BC)) s_tile(j);
    } else {
      if (j >= 1 && !tile_skip((j - 1) * BC)) pv_tile(j - 1);
    }
    // K_{j+1} and V_j must have landed for iteration j+1: only this
    // iteration's copies may remain
    if (ck && cv) FA2_WAIT_VMCNT(2 * IPW);
    else if (ck || cv) FA2_WAIT_VMCNT(IPW);
    else FA2_WAIT_VMCNT(0);
    __syncthreads();
  }

  // ---- epilogue: LSE (S wave), O = O^T / l (PV wave) ------------------------
  if (!pv_role) {
    const float l = sum_halves(l_run);
    if (lh == 0) {
      lslot[lr] = l;
      const __amdgpu_buffer_rsrc_t lr_ = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.lse + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
      const float lse = (m_run + log2f(l)) * 0.69314718055994530942f;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), lr_, (uint32_t)(q * 4), 0, 0);
    }
  }
  __syncthreads();
  if (pv_role) {
    const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((uint16_t*)a.o + head_off), 0, head_bytes, kBufferWord3);
    const float inv = 1.f / lslot[lr];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = E::pack(acc[db][4 * i + 0] * inv, acc[db][4 * i + 1] * inv);
        w[1] = E::pack(acc[db][4 * i + 2] * inv, acc[db][4 * i + 3] * inv);
        const int d = 32 * db + 8 * i + 4 * lh;
        __builtin_amdgcn_raw_buffer_store_b64(w, orr, (uint32_t)(q * KROW + d * 2), 0, 0);
      }
    }
  }
}

}  // namespace fa2
