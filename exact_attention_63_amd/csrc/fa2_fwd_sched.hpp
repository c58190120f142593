// fa2_fwd_sched.hpp -- the scheduled forward kernel for d = 128 (gfx950).
//
// Same method and layouts as fa2_fwd_kernel.hpp ("FlashAttention v2 better
// parallelism + work partitioning" diagram: grid over (batch, head, query
// block), sliced-Q over the waves of a workgroup, online softmax, both
// products on MFMA), with the main loop over full key tiles written out as a
// hand-scheduled assembly block (gen_fwd_sched.py writes it):
//   * 8 waves x 32 query rows, two per SIMD; in the interval of tile j every
//     wave issues the P.V MFMAs of tile j-1 and the score MFMAs of tile j+1,
//     with the softmax of tile j spread between them in staggered rounds, so
//     the matrix pipe is not left idle during the softmax (the overlap of the
//     "FlashAttention v4 Blackwell pipeline co-design" diagram's pseudo-code
//     panel, by software pipelining within each wave);
//   * K/V tiles of 64 keys in a 4-stage LDS ring filled by direct
//     global->LDS copies two tiles ahead, one barrier per tile;
//   * the softmax takes no per-tile max: p = 2^(s c - m) with the row's
//     reference m, and a rare exact update (recompute the tile's scores,
//     new max, rescale) when a lane's row sum exceeds 2^13 -- the
//     conditional rescale of the v4 diagram, in an exact form.
// Tiles that need a mask (crossing the causal diagonal, or past the end of a
// ragged sequence) run a plain C++ loop after the block; the epilogue
// (O = acc / l, LSE) is shared.
//
// The block binds every value it reads or writes to fixed registers: Q
// fragments v[0:31], O^T accumulators v[32:95], m v178, l v179, K fragment
// addresses v[160:167], V^T fragment addresses v[168:175], copy offsets
// v[176:177]; K and V buffer descriptors s[40:43], s[44:47], c s48, tile count
// s49, this wave's LDS copy address s52.  It clobbers v[96:159],
// v[180:FA2_SCHED_REG_END), a few SGPRs, m0, vcc and scc.
#pragma once

#include "fa2_fwd_kernel.hpp"
#include "fa2_fwd_sched.inc"

namespace fa2 {

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x32 __attribute__((ext_vector_type(32)));

// Workgroups of the scheduled kernel cover 256 query rows.
constexpr int kSchedRows = 256;

// LDS reads at a byte address (the kernel's only LDS allocation starts at the
// address the pointer conversion gives; these take that address directly).
__device__ __forceinline__ u32x4 lds_load_b128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)addr;
}
__device__ __forceinline__ u32x2 lds_tr16_at(uint32_t addr) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

template <bool BF16, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fa2_fwd_sched_kernel(Args a) {
  using E = Elem<BF16>;
  constexpr int D = 128, KROW = 2 * D, BC = 64, BR = kSchedRows, NS = 4;
  constexpr int TSZ = BC * KROW;          // bytes of one K (or V) tile
  constexpr int VOFF = NS * TSZ;          // V stages follow the K stages
  constexpr int DK = D / 16, DB = D / 32;
  static_assert(FA2_SCHED_REG_END <= 250, "the loop leaves VGPRs for the compiler");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * NS * TSZ];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  // ---- workgroup -> (query block, head), as in fa2_fwd_kernel ------------
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
  const int q_w = q_wg + wave * 32;

  // key tiles visited, and the leading ones no row of the workgroup masks
  int nt = (N + BC - 1) / BC;
  int nfull = N / BC;
  if constexpr (CAUSAL) {
    nt = min(nt, (min(q_wg + BR, N) - 1) / BC + 1);
    nfull = min(nfull, q_wg / BC);
  }

  // this lane's chunks of the wave's two 1 KiB copy blocks per tile (the LDS
  // chunk p of row r holds the row's logical chunk p ^ chunk_swizzle(r))
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  u32x2v dsrc;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row = (2 * wave + k) * 4 + (lane >> 4);
    dsrc[k] = (uint32_t)(row * KROW + 16 * ((lane & 15) ^ chunk_swizzle<D>(row)));
  }
  // The wave's parts of K of tiles 0-2 and V of tiles 0-1 go to ring stages
  // 0-2 before the Q loads, so that their latencies overlap; the loop waits
  // for them and publishes them with its first barrier (inside the loop,
  // interval j copies K of tile j+3 and V of tile j+2).
  auto copy_half = [&](const __amdgpu_buffer_rsrc_t& r, int region, int tile) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
      lds_dma16(r, smem + region + (tile % NS) * TSZ + (2 * wave + k) * 1024, dsrc[k], tile * TSZ);
  };
  for (int t = 0; t < 3 && t < nfull; ++t) {
    copy_half(kr, 0, t);
    if (t < 2) copy_half(vr, VOFF, t);
  }

  // ---- Q fragments (B operand of S^T = K Q^T), rows past N read as 0 -------
  // Fragment dk is q32[4 dk .. 4 dk + 3].  The main loop and the masked tiles
  // read the same registers (the loop leaves its inputs unchanged).
  u32x32 q32;
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    const u32x4 f = __builtin_amdgcn_raw_buffer_load_b128(qr, (uint32_t)((q_w + lr) * KROW + (2 * dk + lh) * 16), 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) q32[4 * dk + i] = f[i];
  }
  // negative scale folded into Q (c*s = (-c)*(-s) exactly), so c >= 0 below
  const bool c_neg = a.c < 0.f;
  const float c = c_neg ? -a.c : a.c;
  if (c_neg) q32 ^= 0x80008000u;
  auto qfrag = [&](int dk) { return u32x4{q32[4 * dk], q32[4 * dk + 1], q32[4 * dk + 2], q32[4 * dk + 3]}; };

  // ---- LDS addresses (see chunk_swizzle) ----------------------------------
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // K fragment of d step dk: row lr of a 32-key block, chunk 2 dk + lh
  const int kfb = lr * KROW + 16 * (lh ^ chunk_swizzle<D>(lr));
  // V^T fragments through the transpose read: lane (4e + c) of 16-lane group g
  // addresses key row 4 (g/2) + e (+8 for the high half), columns
  // 32 db + 16 (g%2) + 4c
  const int vgq = lane >> 4, ve = (lane >> 2) & 3, vc = lane & 3;
  const int vfb = (4 * (vgq >> 1) + ve) * KROW + 8 * (vc & 1) + 64 * ve +
                  16 * ((2 * (vgq & 1) | (vc >> 1)) ^ (vgq >> 1));
  u32x8 ka, va;
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) ka[dk] = lds0 + (uint32_t)(kfb ^ (32 * dk));
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    va[2 * db] = lds0 + (uint32_t)(VOFF + (vfb ^ (64 * db)));
    va[2 * db + 1] = lds0 + (uint32_t)(VOFF + 8 * KROW + (vfb ^ (64 * db) ^ 32));
  }

  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  float m_run = -INFINITY, l_run = 0.f;

  if (nfull > 0) {
    const uint32_t m0b = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)wave * 2048u);
    const int ntiles = nfull;
#define FA2_SCHED_OPERANDS                                                                                 \
  : "+{v[32:47]}"(acc0), "+{v[48:63]}"(acc1), "+{v[64:79]}"(acc2), "+{v[80:95]}"(acc3), "={v178}"(m_run), \
    "={v179}"(l_run)                                                                                       \
  : "{v[0:31]}"(q32), "{v[160:167]}"(ka), "{v[168:175]}"(va), "{v[176:177]}"(dsrc), "{s[40:43]}"(kr),     \
    "{s[44:47]}"(vr), "{s48}"(c), "{s49}"(ntiles), "{s52}"(m0b)                                            \
  : FA2_SCHED_CLOBBERS
    if constexpr (BF16) asm volatile(FA2_SCHED_BF16 FA2_SCHED_OPERANDS);
    else asm volatile(FA2_SCHED_F16 FA2_SCHED_OPERANDS);
#undef FA2_SCHED_OPERANDS
  }

  // ---- tiles that need a mask: diagonal (causal) or past N (ragged) --------
  if (nfull < nt) {
    __syncthreads();   // the loop's last P.V reads finished in every wave
    for (int j = nfull; j < nt; ++j) {
      const int key0 = j * BC;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        lds_dma16(kr, smem + (2 * wave + k) * 1024, dsrc[k], j * TSZ);
        lds_dma16(vr, smem + VOFF + (2 * wave + k) * 1024, dsrc[k], j * TSZ);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      if (!(CAUSAL && key0 > q_w + 31)) {
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int dk = 0; dk < DK; ++dk)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const u32x4 kf = lds_load_b128(ka[dk] + kb * 32 * KROW);
            s[kb] = E::mfma(kf, qfrag(dk), s[kb]);
          }
        // scale, mask (keys past N, keys after the query), row max
        const int q = q_w + lr;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * lh + (r & 3);
            const bool vis = key < N && (!CAUSAL || key <= q);
            s[kb][r] = vis ? s[kb][r] * c : -INFINITY;
            mx = fmaxf(mx, s[kb][r]);
          }
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;   // never -inf - -inf
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float rs = 0.f;
        u32x4 pf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            float p[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              p[t] = __builtin_amdgcn_exp2f(s[kb][8 * st + t] - m_use);
              rs += p[t];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) pf[kb][st][t] = E::pack(p[2 * t], p[2 * t + 1]);
          }
        l_run = l_run * alpha + rs;
        if (__any(alpha != 1.f)) {
          acc0 *= alpha;
          acc1 *= alpha;
          acc2 *= alpha;
          acc3 *= alpha;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          f32x16& acc = db == 0 ? acc0 : db == 1 ? acc1 : db == 2 ? acc2 : acc3;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
              const int roff = (32 * kb + 16 * st) * KROW;
              const u32x2 lo = lds_tr16_at(va[2 * db] + roff);
              const u32x2 hi = lds_tr16_at(va[2 * db + 1] + roff);
              acc = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kb][st], acc);
            }
        }
      }
      __syncthreads();
    }
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ---------------------
  const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((uint16_t*)a.o + head_off), 0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t lsr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.lse + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
  const int row = q_w + lr;
  const float l = sum_halves(l_run);
  const float inv = 1.f / l;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const f32x16& acc = db == 0 ? acc0 : db == 1 ? acc1 : db == 2 ? acc2 : acc3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = E::pack(acc[4 * i + 0] * inv, acc[4 * i + 1] * inv);
      w[1] = E::pack(acc[4 * i + 2] * inv, acc[4 * i + 3] * inv);
      const int d = 32 * db + 8 * i + 4 * lh;
      __builtin_amdgcn_raw_buffer_store_b64(w, orr, (uint32_t)(row * KROW + d * 2), 0, 0);
    }
  }
  if (lh == 0) {
    const float lse = (m_run + log2f(l)) * 0.69314718055994530942f;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), lsr, (uint32_t)(row * 4), 0, 0);
  }
}

}  // namespace fa2
