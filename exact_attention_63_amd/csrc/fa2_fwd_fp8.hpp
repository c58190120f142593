// fa2_fwd_fp8.hpp -- exact attention forward with FP8 (E4M3) inputs for gfx950.
//
// Method: the tiled online softmax of fa2_fwd_kernel.hpp ("FlashAttention v2
// better parallelism + work partitioning" diagram, concept pseudo-code panel:
// grid over (batch, head, query block), rows split over the waves, per key
// tile S = Q K^T, online softmax update, acc += P V; final O = acc / l from the
// "FlashAttention v4 Blackwell pipeline co-design" diagram).  The v2 diagram's
// panel on what v2 changes names FP8 arithmetic as a capability v2 leaves
// unused; this kernel runs both products on the FP8 matrix cores.
//
// The FP8 scheme (the pages give none):
//   * Q, K and V are OCP E4M3 codes [B, H, N, d], each tensor with one fp32
//     descale factor; O is bf16, LSE fp32.  The descales of Q and K fold into
//     the softmax's exponent scale c = scale * dq * dk * log2(e) (computed on
//     the host in double), the descale of V into the final 1/l.
//   * S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 (fp32 accumulation; the unit
//     E8M0 scale 0x7f leaves the products unscaled).
//   * The reference max of a row moves only when a tile's max exceeds it by
//     more than kFp8Lazy = 0.75 (base 2): the conditional rescale of the v4
//     diagram in its exact form.  P = 2^(c s - m + 8) then never exceeds
//     2^8.75 < 448, and its small values stay out of the E4M3 subnormals down
//     to 2^-14 of the row max.  P is rounded to E4M3 (nearest even,
//     v_cvt_pk_fp8_f32) for O^T += V^T P^T on the same FP8 MFMA; the row sum
//     l takes the fp32 P.  O = acc * (dv / l), LSE = (m + log2 l - 8) ln 2.
//
// Layout (d = 128: 64-key tiles; d = 64: 128-key tiles; one tile of K or V is
// 8 KiB either way, so each of the 8 waves copies 1 KiB of each):
//   * A K tile is [key][d] bytes.  The score MFMA's A operand is 32 bytes of
//     one key row per lane (d in [64s + 32h, +32) for lane half h of d step
//     s), its B operand the same bytes of the lane's query row, held in
//     VGPRs for the whole loop.  Which k slot a byte occupies only has to
//     agree between A and B, and it does: both take the bytes in order.
//   * The S^T accumulator of a 32-key block gives lane (query lr, half h) the
//     keys 8a + 4h + b (a, b in 0..3) in registers 4a + b.  The P.V MFMA's B
//     operand for 64 keys is those 32 values of two blocks packed in register
//     order, so P never leaves the lane.  Its A operand (V^T: d rows, the same
//     keys in the same byte order) comes from the row-major V tile through the
//     gfx950 LDS transpose read ds_read_b64_tr_b8: in each 16-lane group, lane
//     j fetches 8 bytes of row j/2 and receives byte i of all 8 rows, i = its
//     index in the group, which is a column of V.  Four such reads give a lane
//     its 32 keys.
//   * Rows are stored unpadded with their 16-byte chunks XOR-swizzled by
//     fp8_swizzle, so that the 16 key rows of one K fragment read and the
//     8 rows x 2 chunks of one transpose read by 32 lanes fall on distinct
//     banks (blog chapter 4's bank-conflict fix).
//   * Copies go straight from HBM into a 3-stage LDS ring (buffer_load ... lds,
//     one tile ahead of the one in use), with the tile offset in the per-lane
//     offset so that rows past N are range-checked to zero.
#pragma once

#include "fa2_fwd_kernel.hpp"

namespace fa2 {

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct Fp8Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;      // B*H
  int N;       // sequence length
  int nqb;     // query blocks per head
  float c;     // scale * descale_q * descale_k * log2(e)
  float dv;    // descale of V
};

constexpr int kFp8Rows = 256;        // query rows per workgroup (8 waves x 32)
constexpr int kFp8TileBytes = 8192;  // one K (or V) tile: 8192 / d keys
constexpr float kFp8Lazy = 0.75f;    // reference threshold, base 2
constexpr float kFp8Shift = 8.f;     // P is scaled by 2^8 before rounding to E4M3

// XOR swizzle of the 16-byte chunks of a [key][d] row of d bytes (d = 128: 8
// chunks, d = 64: 4 chunks).  d = 128: bits 1, 3, 2 of the row give bits 1, 2,
// 0 of the swizzle, so the 8 rows of one parity among 16 consecutive rows get
// 8 distinct swizzles (K reads) and rows {0,2,8,10} + 4h get swizzles of one
// parity (transpose reads of two adjacent chunks).  d = 64: bits 2 and 3.
template <int D>
__device__ __forceinline__ int fp8_swizzle(int row) {
  if constexpr (D == 128) {
    return (row & 2) | ((row >> 1) & 4) | ((row >> 2) & 1);
  } else {
    static_assert(D == 64, "d must be 64 or 128");
    return (row >> 2) & 3;
  }
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
}

// ds_read_b64_tr_b8 (see the layout notes above)
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* p) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// 16 bytes per lane from a buffer straight into LDS at byte lds + 16 * lane
// (buffer_load_dwordx4 ... lds; out-of-range lanes write zeros).  lds is a
// wave-uniform LDS byte address; the compiler does not track the copy, so the
// kernel orders it itself (s_waitcnt vmcnt, then a barrier).  One wait state
// separates the write of M0 from the copy.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(r)
               : "memory", "m0");
}

// An empty statement that reads x: the value must be computed here.  Kept in
// device-only functions: in the kernel body, an asm operand wider than 16
// bytes makes the host compilation pass drop the kernel's launch stub.
__device__ __forceinline__ void use_vgprs(const f32x16& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void use_vgprs(const i32x8& x) { asm volatile("" ::"v"(x)); }

// four fp32 -> four E4M3 bytes in order (round to nearest even)
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fa2_fwd_fp8_kernel(Fp8Args a) {
  constexpr int TSZ = kFp8TileBytes;
  constexpr int BR = kFp8Rows;
  constexpr int BC = TSZ / D;        // keys per tile
  constexpr int KB = BC / 32;        // 32-key blocks per tile
  constexpr int KS = D / 64;         // 64-wide d steps of the score product
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int PS = BC / 64;        // 64-key steps of the P.V product
  constexpr int NS = 3;              // ring stages
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * NS * TSZ];   // K stages, then V stages

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  // ---- workgroup -> (query block, head), as the 16-bit kernels ------------
  int bh, qblk;
  {
    const int i = blockIdx.x;
    const int total = a.nqb * a.BH;
    if constexpr (!CAUSAL) {
      const int logical = (total % 8 == 0) ? (i % 8) * (total / 8) + i / 8 : i;
      bh = logical / a.nqb;
      qblk = logical % a.nqb;
    } else {
      causal_item(i, a.BH, a.nqb, bh, qblk);
    }
  }
  const int N = a.N;
  const size_t head_off = (size_t)bh * (size_t)N * D;   // elements (= bytes of the inputs)
  const uint32_t head_bytes = (uint32_t)N * D;
  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)a.q + head_off), 0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)a.k + head_off), 0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)a.v + head_off), 0, head_bytes, kBufferWord3);

  const int q_wg = qblk * BR;
  const int q_w = q_wg + wave * 32;          // first query row of this wave
  int nt = (N + BC - 1) / BC;
  if constexpr (CAUSAL) {
    const int last_row = min(q_wg + BR, N) - 1;
    nt = min(nt, last_row / BC + 1);
  }

  // ---- Q fragments: B operand of S^T = K Q^T, kept in VGPRs --------------
  i32x8 qf[KS];
  {
    const uint32_t qoff = (uint32_t)((q_w + lr) * D + 32 * lh);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + 64 * s, 0, 0);
      const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + 64 * s + 16, 0, 0);
      qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }

  // ---- per-row state (base 2) --------------------------------------------
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  // A negative c flips the sign bit of every Q code (exact), so c >= 0 below.
  const bool c_neg = a.c < 0.f;
  const float c = c_neg ? -a.c : a.c;
  if (c_neg) {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] ^= (int)0x80808080u;
  }

  // ---- copies: wave w moves bytes [1024 w, 1024 w + 1024) of each tile -----
  uint32_t dsrc;
  {
    const int b = wave * 1024 + 16 * lane;
    const int row = b / D, phys = (b % D) / 16;
    dsrc = (uint32_t)(row * D + 16 * (phys ^ fp8_swizzle<D>(row)));
  }
  // LDS byte address of this wave's 1 KiB of stage 0 (wave-uniform)
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem + (uint32_t)wave * 1024u);
  auto dma = [&](int tile, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    const uint32_t off = dsrc + (uint32_t)tile * TSZ;
    lds_copy16(kr, ldsw + S * TSZ, off);
    lds_copy16(vr, ldsw + (NS + S) * TSZ, off);
  };

  // ---- fragment addresses ---------------------------------------------------
  // K: row 32 kb + lr, chunks 4 s + 2 lh + e (e = 0, 1)
  int ka[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) ka[e] = lr * D + 16 * ((2 * lh + e) ^ fp8_swizzle<D>(lr));
  // V^T: lane j = lane % 16 of group g = lane / 16 reads row
  // 64 u + 16 x + 8 (r / 4) + 4 h + r % 4 (r = j / 2, h = g / 2) at column
  // 32 db + 16 (g % 2) + 8 (j % 2); the swizzle depends on r and h only
  int vb;
  {
    const int g = lane >> 4, j = lane & 15, r = j >> 1;
    const int vrow = 8 * (r >> 2) + 4 * (g >> 1) + (r & 3);
    vb = vrow * D + 16 * ((g & 1) ^ fp8_swizzle<D>(vrow)) + 8 * (j & 1);
  }

  auto tile_skip = [&](int key0) { return CAUSAL && key0 > q_w + 31; };
  auto tile_masked = [&](int key0) { return (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q_w); };

  // ---- one key tile: scores, softmax, P.V -----------------------------------
  auto tile = [&](int j, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    const int key0 = j * BC;
    if (tile_skip(key0)) return;
    const uint8_t* ks = smem + S * TSZ;
    const uint8_t* vs = smem + (NS + S) * TSZ;

    // S^T = K Q^T
    f32x16 sc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sc[kb] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint8_t* kp = ks + 32 * kb * D;
        const u32x4 lo = *(const u32x4*)(kp + (ka[0] ^ (64 * s)));
        const u32x4 hi = *(const u32x4*)(kp + (ka[1] ^ (64 * s)));
        const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sc[kb] = mfma_fp8(kf, qf[s], sc[kb]);
      }
    }
    // keep the phases apart: hoisting the P.V operand reads above the softmax
    // would hold them in registers beside the scores
    __builtin_amdgcn_sched_barrier(0);

    // tile max (base 2)
    float cc = c, m_tile;
    if (tile_masked(key0)) {
      // key key0 + 4 lh + off (off = 32 kb + 8 (r / 4) + r % 4) is visible iff
      // off < lim: one per-lane bound against compile-time offsets
      const int lim = (CAUSAL ? min(N, q_w + lr + 1) : N) - key0 - 4 * lh;
      float e0 = -INFINITY, e1 = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool vis = 32 * kb + 8 * (r >> 2) + (r & 3) < lim;
          const float t = vis ? sc[kb][r] * c : -INFINITY;
          sc[kb][r] = t;
          if (r & 1) e1 = fmaxf(e1, t); else e0 = fmaxf(e0, t);
        }
      m_tile = max_halves(fmaxf(e0, e1));
      cc = 1.f;
    } else {
      float e0 = sc[0][0], e1 = sc[0][1];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          e0 = fmaxf(e0, fmaxf(sc[kb][r], sc[kb][r + 1]));
          e1 = fmaxf(e1, fmaxf(sc[kb][r + 2], sc[kb][r + 3]));
        }
      m_tile = max_halves(fmaxf(e0, e1)) * c;
    }
    const float m_old = m_run;
    const float m_new = (m_tile > m_old + kFp8Lazy) ? m_tile : m_old;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_old - m_use);
    m_run = m_new;
    const float ref = m_use - kFp8Shift;

    // P = 2^(c s - ref), row sum over fp32 P, E4M3 for the product
    i32x8 pk[PS];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][4 * w + t], cc, -ref));
          if (t & 1) rs1 += p[t]; else rs0 += p[t];
        }
        pk[kb >> 1][4 * (kb & 1) + w] = (int)pack_fp8x4(p[0], p[1], p[2], p[3]);
      }
    }
    l_run = l_run * alpha + (rs0 + rs1);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }

    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T
#pragma unroll
    for (int u = 0; u < PS; ++u) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        i32x8 vf;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const u32x2 t = lds_read_tr8(vs + (64 * u + 16 * x) * D + (vb ^ (32 * db)));
          vf[2 * x] = (int)t[0];
          vf[2 * x + 1] = (int)t[1];
        }
        acc[db] = mfma_fp8(vf, pk[u], acc[db]);
      }
    }
    // an explicit use keeps the compiler from sinking these products into
    // the next tile, past its scores, with P and V^T held live meanwhile
#pragma unroll
    for (int db = 0; db < DB; ++db) use_vgprs(acc[db]);
  };

  auto step = [&](int j, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;    // == j % NS
    // this wave's copies of tile j are complete once at most those of tile
    // j + 1 (two instructions) remain
    if (j + 1 < nt) FA2_WAIT_VMCNT(2); else FA2_WAIT_VMCNT(0);
    // every wave's copies of tile j have landed and every wave is done with
    // tile j - 1, whose stage the copy of tile j + 2 refills
    __syncthreads();
    if (j + NS - 1 < nt) dma(j + NS - 1, std::integral_constant<int, (S + NS - 1) % NS>{});
    tile(j, stage_tag);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  dma(0, I0{});
  if (nt > 1) dma(1, I1{});
  // the Q loads were issued before the copies: wait for them only
  if (nt > 1) FA2_WAIT_VMCNT(4); else FA2_WAIT_VMCNT(2);
#pragma unroll
  for (int s = 0; s < KS; ++s) use_vgprs(qf[s]);
  int j = 0;
  for (; j + NS <= nt; j += NS) {
    step(j, I0{});
    step(j + 1, I1{});
    step(j + 2, I2{});
  }
  if (j < nt) step(j, I0{});
  if (j + 1 < nt) step(j + 1, I1{});

  // ---- epilogue: O = acc * (dv / l) in bf16, LSE = (m + log2 l - 8) ln 2 -----
  const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((uint16_t*)a.o + head_off), 0, head_bytes * 2u, kBufferWord3);
  const __amdgpu_buffer_rsrc_t lsr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.lse + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
  const int row = q_w + lr;
  const float l = sum_halves(l_run);
  const float sc_o = a.dv / l;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = Elem<true>::pack(acc[db][4 * i + 0] * sc_o, acc[db][4 * i + 1] * sc_o);
      w[1] = Elem<true>::pack(acc[db][4 * i + 2] * sc_o, acc[db][4 * i + 3] * sc_o);
      const int d = 32 * db + 8 * i + 4 * lh;
      __builtin_amdgcn_raw_buffer_store_b64(w, orr, (uint32_t)(row * D * 2 + d * 2), 0, 0);
    }
  }
  if (lh == 0) {
    const float lse = (m_run + log2f(l) - kFp8Shift) * 0.69314718055994530942f;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), lsr, (uint32_t)(row * 4), 0, 0);
  }
}

}  // namespace fa2
