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
//     more than kFp8Lazy = 2.75 (base 2): the conditional rescale of the v4
//     diagram in its exact form.  P = 2^(c s - m + 6) then never exceeds
//     2^8.75 < 448, and its values down to 2^-12 of the reference stay normal
//     E4M3 numbers; a group of 32 rows rescales acc in about 6 % of the
//     tiles of N(0,1) inputs (about half with a shift of 8 and a threshold of
//     0.75).  P is rounded to E4M3 (nearest even, v_cvt_pk_fp8_f32) for
//     O^T += V^T P^T on the same FP8 MFMA; the row sum l takes the fp32 P.
//     O = acc * (dv / l), LSE = (m + log2 l - 6) ln 2.
//
// Layout (d = 128: 64-key tiles; d = 64: 128-key tiles; one tile of K or V is
// 8 KiB either way, copied in 1 KiB blocks by the waves of the workgroup):
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

constexpr int kFp8TileBytes = 8192;  // one K (or V) tile: 8192 / d keys
constexpr float kFp8Lazy = 2.75f;    // reference threshold, base 2
constexpr float kFp8Shift = 6.f;     // P is scaled by 2^6 before rounding to E4M3

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
  // the first conversion's other half is overwritten by the second one
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <int D, int NW>
struct Fp8Geom {
  static constexpr int TSZ = kFp8TileBytes;
  static constexpr int BR = NW * 32;   // query rows per workgroup (NW waves x 32)
  static constexpr int CPW = 8 / NW;   // 1 KiB copy blocks per wave, tile and tensor
  static constexpr int BC = TSZ / D;   // keys per tile
  static constexpr int KB = BC / 32;   // 32-key blocks per tile
  static constexpr int KS = D / 64;    // 64-wide d steps of the score product
  static constexpr int DB = D / 32;    // 32-row blocks of O^T
  static constexpr int PS = BC / 64;   // 64-key steps of the P.V product
};

// One wave's view of a workgroup: its head, rows, Q fragments, online-softmax
// state and fragment addresses.  The kernels below differ only in how they
// order the steps of the loop over key tiles.
template <int D, bool CAUSAL, int NW>
struct Fp8Wave {
  using G = Fp8Geom<D, NW>;
  __amdgpu_buffer_rsrc_t kr, vr;
  int bh, N, q_wg, q_w, nt, lr, lh;
  float c;                 // |scale * dq * dk * log2(e)|
  i32x8 qf[G::KS];         // B operand of S^T = K Q^T
  f32x16 acc[G::DB];       // O^T
  float m_run, l_run;      // reference max and row sum (base 2, P scaled by 2^6)
  uint32_t dsrc[G::CPW];   // copy source offsets in a tile
  uint32_t ldsw;           // this wave's LDS destination in a stage
  int ka[2], vb;           // K and V^T fragment addresses inside a stage

  __device__ __forceinline__ void init(const Fp8Args& a, uint8_t* smem) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    lr = lane & 31;
    lh = lane >> 5;
    int qblk;
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
    N = a.N;
    const size_t head_off = (size_t)bh * (size_t)N * D;   // elements = bytes of the inputs
    const uint32_t head_bytes = (uint32_t)N * D;
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)a.q + head_off), 0, head_bytes, kBufferWord3);
    kr = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.k + head_off), 0, head_bytes, kBufferWord3);
    vr = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.v + head_off), 0, head_bytes, kBufferWord3);
    q_wg = qblk * G::BR;
    q_w = q_wg + wave * 32;
    nt = (N + G::BC - 1) / G::BC;
    if constexpr (CAUSAL) nt = min(nt, (min(q_wg + G::BR, N) - 1) / G::BC + 1);

    // Q: bytes [64 s + 32 lh, +32) of query row q_w + lr
    const uint32_t qoff = (uint32_t)((q_w + lr) * D + 32 * lh);
#pragma unroll
    for (int s = 0; s < G::KS; ++s) {
      const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + 64 * s, 0, 0);
      const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + 64 * s + 16, 0, 0);
      qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    // a negative c flips the sign bit of every Q code (exact), so c >= 0 below
    c = a.c;
    if (c < 0.f) {
      c = -c;
#pragma unroll
      for (int s = 0; s < G::KS; ++s) qf[s] ^= (int)0x80808080u;
    }
#pragma unroll
    for (int db = 0; db < G::DB; ++db) acc[db] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;

    // copies: wave w moves bytes [1024 CPW w, 1024 CPW (w + 1)) of each tile
#pragma unroll
    for (int k = 0; k < G::CPW; ++k) {
      const int b = (wave * G::CPW + k) * 1024 + 16 * lane;
      const int row = b / D, phys = (b % D) / 16;
      dsrc[k] = (uint32_t)(row * D + 16 * (phys ^ fp8_swizzle<D>(row)));
    }
    ldsw = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem +
                                          (uint32_t)(wave * G::CPW) * 1024u);
    // K: row 32 kb + lr, chunks 4 s + 2 lh + e (e = 0, 1)
#pragma unroll
    for (int e = 0; e < 2; ++e) ka[e] = lr * D + 16 * ((2 * lh + e) ^ fp8_swizzle<D>(lr));
    // V^T: lane j = lane % 16 of group g = lane / 16 reads row
    // 64 u + 16 x + 8 (r / 4) + 4 h + r % 4 (r = j / 2, h = g / 2) at column
    // 32 db + 16 (g % 2) + 8 (j % 2); the swizzle depends on r and h only
    {
      const int g = lane >> 4, j = lane & 15, r = j >> 1;
      const int vrow = 8 * (r >> 2) + 4 * (g >> 1) + (r & 3);
      vb = vrow * D + 16 * ((g & 1) ^ fp8_swizzle<D>(vrow)) + 8 * (j & 1);
    }
  }

  // this wave's share of one tile's K (or V) copy into the LDS stage at byte
  // offset stage_off: CPW instructions
  __device__ __forceinline__ void copy(__amdgpu_buffer_rsrc_t r, int tile, uint32_t stage_off) const {
#pragma unroll
    for (int k = 0; k < G::CPW; ++k) lds_copy16(r, ldsw + stage_off + 1024 * k, dsrc[k] + (uint32_t)tile * G::TSZ);
  }

  __device__ __forceinline__ bool masked(int key0) const {
    return (key0 + G::BC > N) || (CAUSAL && key0 + G::BC - 1 > q_w);
  }

  // one 32-key block of S^T = K Q^T from the K tile at ks
  __device__ __forceinline__ void score_block(const uint8_t* ks, int kb, f32x16& sb) const {
    sb = f32x16{};
#pragma unroll
    for (int s = 0; s < G::KS; ++s) {
      const uint8_t* kp = ks + 32 * kb * D;
      const u32x4 lo = *(const u32x4*)(kp + (ka[0] ^ (64 * s)));
      const u32x4 hi = *(const u32x4*)(kp + (ka[1] ^ (64 * s)));
      const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      sb = mfma_fp8(kf, qf[s], sb);
    }
  }

  // S^T = K Q^T from the K tile at ks
  __device__ __forceinline__ void scores(const uint8_t* ks, f32x16 (&sc)[G::KB]) const {
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb) sc[kb] = f32x16{};
#pragma unroll
    for (int s = 0; s < G::KS; ++s) {
#pragma unroll
      for (int kb = 0; kb < G::KB; ++kb) {
        const uint8_t* kp = ks + 32 * kb * D;
        const u32x4 lo = *(const u32x4*)(kp + (ka[0] ^ (64 * s)));
        const u32x4 hi = *(const u32x4*)(kp + (ka[1] ^ (64 * s)));
        const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sc[kb] = mfma_fp8(kf, qf[s], sc[kb]);
      }
    }
  }

  // online softmax of one tile of scores (keys from key0), in two parts.
  // ref_update: masks the scores (MASKED), takes the tile max, moves the
  // reference when the max exceeds it by more than kFp8Lazy, and returns
  // alpha = 2^(m_old - m_new), the multiplier cc of the stored scores and
  // the subtrahend ref of the exponent (P is scaled by 2^6).
  template <bool MASKED>
  __device__ __forceinline__ void ref_update(f32x16 (&sc)[G::KB], int key0, float& alpha, float& cc, float& ref) {
    float m_tile;
    cc = c;
    if constexpr (MASKED) {
      // key key0 + 4 lh + off (off = 32 kb + 8 (r / 4) + r % 4) is visible
      // iff off < lim: one per-lane bound against compile-time offsets
      const int lim = (CAUSAL ? min(N, q_w + lr + 1) : N) - key0 - 4 * lh;
      float e0 = -INFINITY, e1 = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < G::KB; ++kb)
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
      for (int kb = 0; kb < G::KB; ++kb)
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
    alpha = __builtin_amdgcn_exp2f(m_old - m_use);
    m_run = m_new;
    ref = m_use - kFp8Shift;
  }
  // exp_block: P = 2^(cc s - ref) of one 32-key block, added to the row sums
  // (fp32) and packed as E4M3 in the B-operand order of the P.V product
  __device__ __forceinline__ void exp_block(const f32x16& s, int kb, float cc, float ref, i32x8 (&pk)[G::PS],
                                            float& rs0, float& rs1) const {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * w + t], cc, -ref));
        if (t & 1) rs1 += p[t]; else rs0 += p[t];
      }
      pk[kb >> 1][4 * (kb & 1) + w] = (int)pack_fp8x4(p[0], p[1], p[2], p[3]);
    }
  }
  // both parts over the whole tile
  template <bool MASKED>
  __device__ __forceinline__ void softmax(f32x16 (&sc)[G::KB], int key0, i32x8 (&pk)[G::PS], float& alpha) {
    float cc, ref, rs0 = 0.f, rs1 = 0.f;
    ref_update<MASKED>(sc, key0, alpha, cc, ref);
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb) exp_block(sc[kb], kb, cc, ref, pk, rs0, rs1);
    l_run = l_run * alpha + (rs0 + rs1);
  }

  // acc *= alpha when some row of the wave moved its reference
  __device__ __forceinline__ void rescale(float alpha) {
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < G::DB; ++db) acc[db] *= alpha;
    }
  }

  // O^T += V^T P^T from the V tile at vs
  __device__ __forceinline__ void pv(const uint8_t* vs, const i32x8 (&pk)[G::PS]) {
#pragma unroll
    for (int u = 0; u < G::PS; ++u) {
#pragma unroll
      for (int db = 0; db < G::DB; ++db) {
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
  }

  // O = acc * (dv / l) in bf16, LSE = (m + log2 l - 6) ln 2.  With d = 128, O
  // goes through this wave's kStageBytes of LDS at stage (store_o128_staged;
  // 4 KiB aligned, no longer read by any wave), else straight from the
  // accumulators.
  __device__ __forceinline__ void store(const Fp8Args& a, uint8_t* stage) const {
    const size_t head_off = (size_t)bh * (size_t)N * D;
    const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((uint16_t*)a.o + head_off), 0, (uint32_t)N * D * 2u, kBufferWord3);
    const __amdgpu_buffer_rsrc_t lsr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.lse + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
    const int row = q_w + lr;
    const float l = sum_halves(l_run);
    const float so = a.dv / l;
    if constexpr (D == 128) {
      store_o128_staged<true>(orr, q_w, lr + 32 * lh, acc[0], acc[1], acc[2], acc[3], so, stage);
    } else {
      (void)stage;
#pragma unroll
      for (int db = 0; db < G::DB; ++db) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 w;
          w[0] = Elem<true>::pack(acc[db][4 * i + 0] * so, acc[db][4 * i + 1] * so);
          w[1] = Elem<true>::pack(acc[db][4 * i + 2] * so, acc[db][4 * i + 3] * so);
          const int d = 32 * db + 8 * i + 4 * lh;
          __builtin_amdgcn_raw_buffer_store_b64(w, orr, (uint32_t)(row * D * 2 + d * 2), 0, 0);
        }
      }
    }
    if (lh == 0) {
      const float lse = (m_run + log2f(l) - kFp8Shift) * 0.69314718055994530942f;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), lsr, (uint32_t)(row * 4), 0, 0);
    }
  }
};

// Tile by tile: S, softmax and P.V of tile j between two barriers, the copy
// of tile j + 2 in flight meanwhile (3-stage ring of K and V tiles).  NW
// waves per workgroup; WPE: waves per SIMD the register budget is sized for.
// With NW = 4 and WPE = 3 (at most 168 VGPRs) three workgroups share a CU and
// their barriers are independent, so one's softmax overlaps another's
// matrix products; with NW = 8 and WPE = 2 one workgroup of 256 rows fills
// it.
template <int D, bool CAUSAL, int NW, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(WPE, WPE)))
void fa2_fwd_fp8_kernel(Fp8Args a) {
  using G = Fp8Geom<D, NW>;
  constexpr int TSZ = G::TSZ, NS = 3, CPW = G::CPW;
  __shared__ __attribute__((aligned(4096))) uint8_t smem[2 * NS * TSZ];   // K stages, then V stages
  static_assert(NW * kStageBytes <= 2 * NS * TSZ, "the ring holds the output staging");
  Fp8Wave<D, CAUSAL, NW> w;
  w.init(a, smem);
  const int nt = w.nt;

  auto tile = [&](int j, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    const int key0 = j * G::BC;
    if (CAUSAL && key0 > w.q_w + 31) return;     // above this wave's diagonal
    f32x16 sc[G::KB];
    i32x8 pk[G::PS];
    float alpha;
    w.scores(smem + S * TSZ, sc);
    // keep the phases apart: hoisting the P.V operand reads above the softmax
    // would hold them in registers beside the scores
    __builtin_amdgcn_sched_barrier(0);
    if (w.masked(key0)) w.template softmax<true>(sc, key0, pk, alpha);
    else w.template softmax<false>(sc, key0, pk, alpha);
    w.rescale(alpha);
    __builtin_amdgcn_sched_barrier(0);
    w.pv(smem + (NS + S) * TSZ, pk);
    // an explicit use keeps the compiler from sinking these products into
    // the next tile, past its scores, with P and V^T held live meanwhile
#pragma unroll
    for (int db = 0; db < G::DB; ++db) use_vgprs(w.acc[db]);
  };
  auto step = [&](int j, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;    // == j % NS
    // this wave's copies of tile j are complete once at most those of tile
    // j + 1 (2 CPW instructions) remain
    if (j + 1 < nt) FA2_WAIT_VMCNT(2 * CPW); else FA2_WAIT_VMCNT(0);
    // every wave's copies of tile j have landed and every wave is done with
    // tile j - 1, whose stage the copy of tile j + 2 refills
    __syncthreads();
    if (j + NS - 1 < nt) {
      constexpr int S2 = (S + NS - 1) % NS;
      w.copy(w.kr, j + NS - 1, S2 * TSZ);
      w.copy(w.vr, j + NS - 1, (NS + S2) * TSZ);
    }
    tile(j, stage_tag);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  w.copy(w.kr, 0, 0);
  w.copy(w.vr, 0, NS * TSZ);
  if (nt > 1) {
    w.copy(w.kr, 1, TSZ);
    w.copy(w.vr, 1, (NS + 1) * TSZ);
  }
  // the Q loads were issued before the copies: wait for them only
  if (nt > 1) FA2_WAIT_VMCNT(4 * CPW); else FA2_WAIT_VMCNT(2 * CPW);
#pragma unroll
  for (int s = 0; s < G::KS; ++s) use_vgprs(w.qf[s]);
  int j = 0;
  for (; j + NS <= nt; j += NS) {
    step(j, I0{});
    step(j + 1, I1{});
    step(j + 2, I2{});
  }
  if (j < nt) step(j, I0{});
  if (j + 1 < nt) step(j + 1, I1{});
  if constexpr (D == 128) {
    __syncthreads();   // every wave is done with the ring: it stages the output
    w.store(a, smem + (threadIdx.x >> 6) * kStageBytes);
  } else {
    w.store(a, nullptr);
  }
}

}  // namespace fa2
