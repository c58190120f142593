// fa2_bwd_kernel.hpp -- exact attention backward for gfx950 (CDNA4): dQ, dK
// and dV from Q, K, V, O, the forward pass's LSE and the upstream gradient dO.
//
// Method.  The pages name the backward pass as the step that follows the
// forward one ("FlashAttention v4 Blackwell pipeline co-design" diagram: its
// list of v4 directions and its backward note aim at removing the atomic
// accumulation of dQ) but print no formulas; the gradients are those of the
// forward definition.  With S = scale * Q K^T (masked), P = softmax rows of
// S (recomputed from the saved LSE: P = exp(S - LSE), so no N x N matrix is
// ever stored, as in the forward pass), O = P V and the upstream gradient dO:
//
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_t dO_it O_it,
//   dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three kernels, all enqueued on the caller's stream:
//   * fa2_bwd_delta_kernel: D_i = dO_i . O_i (fp32), one row per 8 or 16
//     lanes, written to the caller's delta buffer;
//   * dK/dV: one workgroup per (key block, head); 32 keys per wave or per
//     pair of waves (the sliced-Q split of the forward pass, with keys in the
//     place of queries); K, V rows in VGPRs, dK^T, dV^T accumulators in
//     registers; the query tiles (Q, dO, LSE and D) walk through LDS.  Three
//     configurations: fa2_bwd_dkdv_kernel (each wave accumulates both, one
//     wave per SIMD), fa2_bwd_dkdv_pair_kernel (the dV wave hands P to the
//     dK wave through LDS, so every product is computed once) and
//     fa2_bwd_dkdv_pipe_kernel (the same hand-off pipelined across query
//     tiles);
//   * fa2_bwd_dq_kernel: one workgroup per (query block, head); each wave
//     owns 32 queries, keeps their Q and dO rows in VGPRs and the dQ^T
//     accumulator in registers, and walks the key tiles (K, V in LDS);
//     option: a fixed MFMA issue order (LOOK).
// dQ is thus produced by its own partition of the work, not by atomic adds
// across key blocks: the result is deterministic and needs no workspace, at
// the cost of recomputing S and dP in the dQ kernel.
//
// MFMA layouts (v_mfma_f32_32x32x16, 16-bit inputs, fp32 accumulation).  A
// 32x32 result block leaves column (lane % 32) in each lane and rows
// 8*(r/4) + 4*(lane/32) + r%4 in its registers r = 0..15.  The dK/dV kernel
// computes S = Q K_w^T and dP = dO V_w^T with the wave's keys as columns, so
// P and dS are exactly the B operands of dV^T += dO^T P and dK^T += Q^T dS
// once queries are renumbered inside each 32-query block (as the forward pass
// renumbers keys); dO^T and Q^T come from the row-major LDS tiles through the
// transpose read ds_read_b64_tr_b16, whose lane mapping realises that
// renumbering.  The dQ kernel is the forward pass's layout: S^T = K Q_w^T,
// dP^T = V dO_w^T (queries as columns), dQ^T += K^T dS^T.
//
// LDS tiles are unpadded rows whose 16-byte chunks are XOR-swizzled
// (chunk_swizzle): 16-byte fragment reads and transpose reads of one tile
// both fall on distinct banks.  Global reads and writes are buffer
// instructions bounded by the head's extent: rows past N read as zero and
// their stores are dropped.
#pragma once

#include "fa2_fwd_kernel.hpp"

namespace fa2 {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  int BH;       // B*H
  int N;        // sequence length
  int nblk;     // key blocks (dK/dV kernel) or query blocks (dQ kernel) per head
  float c;      // scale * log2(e)
  float scale;
};

// Workgroup shape of the dK/dV and dQ kernels: NW waves of 32 rows each,
// built for WPE waves per SIMD.
template <int NW_, int WPE_>
struct BwdTile {
  static constexpr int NW = NW_, WPE = WPE_;
  static constexpr int THREADS = NW * 64;
  static constexpr int BR = 32 * NW;   // keys (dK/dV) or queries (dQ) per workgroup
};

constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// the two 16-bit halves of a packed word as fp32
template <bool BF16>
__device__ __forceinline__ float half_lo(uint32_t w) {
  if constexpr (BF16) {
    return __builtin_bit_cast(float, w << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  }
}
template <bool BF16>
__device__ __forceinline__ float half_hi(uint32_t w) {
  if constexpr (BF16) {
    return __builtin_bit_cast(float, w & 0xFFFF0000u);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
}

// ---------------------------------------------------------------------------
// D_i = sum_t dO[i, t] * O[i, t] in fp32.  Each lane takes one 16-byte chunk
// (8 elements) of a row; the D/8 lanes of a row (8 or 16 consecutive lanes)
// combine their partial sums with lane exchanges.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void fa2_bwd_delta_kernel(BwdArgs a, long long rows) {
  constexpr int CPR = D / 8;
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = g / CPR;
  const int ch = (int)(g % CPR);
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + (size_t)ch * 8;
    const u32x4 x = *(const u32x4*)((const uint16_t*)a.o + off);
    const u32x4 y = *(const u32x4*)((const uint16_t*)a.dout + off);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = __builtin_fmaf(half_lo<BF16>(x[t]), half_lo<BF16>(y[t]), acc);
      acc = __builtin_fmaf(half_hi<BF16>(x[t]), half_hi<BF16>(y[t]), acc);
    }
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && ch == 0) a.delta[row] = acc;
}

// 4 bytes per lane from a buffer straight into LDS (lane l writes lds + 4*l),
// as inline assembly like lds_dma16_asm: invisible to the compiler's wait
// counting, so the kernel's own s_waitcnt vmcnt and barriers order it.
__device__ __forceinline__ void lds_dma4_asm(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voffset,
                                             int soffset) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(dst), "v"(voffset), "s"(r), "s"(soffset)
               : "memory", "m0");
}

// LDS byte offsets of a lane's operand fragments in an unpadded, swizzled
// [row][D] tile (see chunk_swizzle):
//   frag_base: 16-byte read of row (lane % 32), chunk 2*dk + lane/32, for the
//     A operand of a product whose k dimension is d; XOR with 32*dk selects
//     the d step, add 32*KROW per 32-row block;
//   trans_base: the two transpose reads of the A operand whose k dimension
//     runs over the tile's rows (16 renumbered rows per step) and whose m
//     dimension is d (32-wide block db): element i%4 of the 8 bytes that
//     lane 4e + i/4 of a 16-lane group loads lands in output lane i.
template <int D>
struct FragAddr {
  static constexpr int KROW = D * 2;
  int frag;          // frag_base
  int trans[D / 32][2];
  __device__ __forceinline__ explicit FragAddr(int lane) {
    const int lr = lane & 31, lh = lane >> 5;
    frag = lr * KROW + 16 * (lh ^ chunk_swizzle<D>(lr));
    const int g = lane >> 4, e = (lane >> 2) & 3, c = lane & 3;
    const int tb = (4 * (g >> 1) + e) * KROW + 8 * (c & 1) + (D == 128 ? 64 * e : 64 * (e >> 1)) +
                   16 * ((2 * (g & 1) | (c >> 1)) ^ (g >> 1));
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      trans[db][0] = tb ^ (64 * db);
      trans[db][1] = 8 * KROW + (tb ^ (64 * db) ^ 32);
    }
  }
  // A operand (m = d block db, k = 16 tile rows starting at row0) from the tile at lds
  __device__ __forceinline__ u32x4 tread(const uint8_t* lds, int row0, int db) const {
    const u32x2 lo = lds_read_tr16(lds + trans[db][0] + row0 * KROW);
    const u32x2 hi = lds_read_tr16(lds + trans[db][1] + row0 * KROW);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
  // A operand (m = 32 rows starting at row0, k = d step dk)
  __device__ __forceinline__ u32x4 fread(const uint8_t* lds, int row0, int dk) const {
    return *(const u32x4*)(lds + (frag ^ (32 * dk)) + row0 * KROW);
  }
};

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (key block of 32*NW keys, head), wave w owns keys
// [k_wg + 32w, +32).  Query tiles of 64 rows: Q, dO (row-major, swizzled),
// LSE (base 2) and D staged in LDS, two stages, register-staged copies.
template <bool BF16, int D, bool CAUSAL, class TL>
__global__ __attribute__((amdgpu_flat_work_group_size(TL::THREADS, TL::THREADS),
                          amdgpu_waves_per_eu(TL::WPE, TL::WPE)))
void fa2_bwd_dkdv_kernel(BwdArgs a) {
  using E = Elem<BF16>;
  constexpr int T = TL::THREADS, BK = TL::BR;
  constexpr int BQ = 64;                    // queries per tile
  constexpr int NQB = BQ / 32;              // 32-query blocks per tile
  constexpr int DK = D / 16, DB = D / 32, KROW = D * 2;
  constexpr int TSZ = BQ * KROW;            // bytes of one Q (or dO) tile
  constexpr int STAGE = 2 * TSZ + 2 * BQ * 4;
  constexpr int CH = BQ * D / 8;            // 16-byte chunks per tile
  constexpr int CH_T = CH / T;
  static_assert(CH % T == 0, "tile copy must split evenly over threads");
  static_assert(T >= 2 * BQ, "LSE and D rows need 2*BQ threads");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;

  int bh, kblk;
  {
    const int i = blockIdx.x;
    const int total = a.nblk * a.BH;
    if constexpr (!CAUSAL) {
      // consecutive logical ids (the key blocks of one head) on one XCD
      const int logical = (total % 8 == 0) ? (i % 8) * (total / 8) + i / 8 : i;
      bh = logical / a.nblk;
      kblk = logical % a.nblk;
    } else {
      // key block 0 sees every query: heaviest first
      bh = i % a.BH;
      kblk = i / a.BH;
    }
  }
  const int N = a.N;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  auto rsrc = [&](const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p + head_off), 0, head_bytes, kBufferWord3);
  };
  const __amdgpu_buffer_rsrc_t qr = rsrc(a.q), kr = rsrc(a.k), vr = rsrc(a.v), dor = rsrc(a.dout);
  const __amdgpu_buffer_rsrc_t lser = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.lse + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t dlr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.delta + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);

  const int k_wg = kblk * BK;
  const int k_w = k_wg + 32 * wave;
  const int key = k_w + lr;                 // this lane's key (column of S, P, dP, dS)

  // K and V rows of the wave's keys: B operands (k = d step dk), kept in VGPRs
  u32x4 kf[DK], vf[DK];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    const uint32_t off = (uint32_t)(key * KROW + (2 * dk + lh) * 16);
    kf[dk] = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
    vf[dk] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
  }
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }

  // query tiles this workgroup visits
  const int nt = (N + BQ - 1) / BQ;
  const int t0 = CAUSAL ? k_wg / BQ : 0;

  u32x4 qst[CH_T], dost[CH_T];
  float lst = 0.f;
  auto load = [&](int q0) {
#pragma unroll
    for (int it = 0; it < CH_T; ++it) {
      const int e = tid + it * T;
      const int row = e / (D / 8), ch = e % (D / 8);
      const uint32_t off = (uint32_t)((q0 + row) * KROW + ch * 16);
      qst[it] = __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0);
      dost[it] = __builtin_amdgcn_raw_buffer_load_b128(dor, off, 0, 0);
    }
    if (tid < BQ) {
      lst = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lser, (uint32_t)((q0 + tid) * 4), 0, 0));
    } else if (tid < 2 * BQ) {
      lst = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dlr, (uint32_t)((q0 + tid - BQ) * 4), 0, 0));
    }
  };
  auto store = [&](int stg) {
    uint8_t* base = smem + stg * STAGE;
#pragma unroll
    for (int it = 0; it < CH_T; ++it) {
      const int e = tid + it * T;
      const int row = e / (D / 8), ch = e % (D / 8);
      const int off = row * KROW + 16 * (ch ^ chunk_swizzle<D>(row));
      *(u32x4*)(base + off) = qst[it];
      *(u32x4*)(base + TSZ + off) = dost[it];
    }
    // LSE in base 2, then D
    if (tid < BQ) {
      ((float*)(base + 2 * TSZ))[tid] = lst * kLog2e;
    } else if (tid < 2 * BQ) {
      ((float*)(base + 2 * TSZ))[tid] = lst;
    }
  };

  const FragAddr<D> fa(lane);
  const float c = a.c;

  auto compute = [&](const uint8_t* st, int q0, bool masked) {
    const uint8_t* qt = st;
    const uint8_t* dot = st + TSZ;
    const float* l2 = (const float*)(st + 2 * TSZ);
    const float* dl = l2 + BQ;
    // S = Q K_w^T and dP = dO V_w^T: queries as rows, the wave's keys as columns
    f32x16 s[NQB], dp[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
    }
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        s[qb] = E::mfma(fa.fread(qt, 32 * qb, dk), kf[dk], s[qb]);
        dp[qb] = E::mfma(fa.fread(dot, 32 * qb, dk), vf[dk], dp[qb]);
      }
    }
    // P = 2^(s*c - LSE2), dS = P * (dP - D); both packed to 16 bits as the B
    // operands of the two products below (registers [8st, 8st+8) = 16-query step st)
    u32x4 pp[NQB][2], dsp[NQB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      f32x4 lq[4], dq[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        lq[g] = *(const f32x4*)(l2 + 32 * qb + 8 * g + 4 * lh);
        dq[g] = *(const f32x4*)(dl + 32 * qb + 8 * g + 4 * lh);
      }
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float lv = lq[r >> 2][r & 3], dv = dq[r >> 2][r & 3];
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], c, -lv));
        if (masked) {
          const int q = q0 + 32 * qb + 8 * (r >> 2) + 4 * lh + (r & 3);
          const bool vis = q < N && (!CAUSAL || key <= q);
          pv = vis ? pv : 0.f;
        }
        p[r] = pv;
        ds[r] = pv * (dp[qb][r] - dv);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          pp[qb][h][t] = E::pack(p[8 * h + 2 * t], p[8 * h + 2 * t + 1]);
          dsp[qb][h][t] = E::pack(ds[8 * h + 2 * t], ds[8 * h + 2 * t + 1]);
        }
    }
    // dV^T += dO^T P, dK^T += Q^T dS (k = 16 renumbered queries per step)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          dva[db] = E::mfma(fa.tread(dot, 32 * qb + 16 * h, db), pp[qb][h], dva[db]);
          dka[db] = E::mfma(fa.tread(qt, 32 * qb + 16 * h, db), dsp[qb][h], dka[db]);
        }
  };

  if (t0 < nt) {
    load(t0 * BQ);
    store(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    for (int t = t0; t < nt; ++t) {
      const int q0 = t * BQ;
      const int stg = (t - t0) & 1;
      if (t + 1 < nt) load(q0 + BQ);
      // all of this tile's queries precede all of the wave's keys: nothing visible
      const bool skip = CAUSAL && q0 + BQ - 1 < k_w;
      if (!skip) {
        const bool masked = (q0 + BQ > N) || (CAUSAL && q0 < k_w + 31);
        compute(smem + stg * STAGE, q0, masked);
      }
      if (t + 1 < nt) store(stg ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: dK = scale * dK^T (transposed back), dV = dV^T -----------
  const __amdgpu_buffer_rsrc_t dkr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((uint16_t*)a.dk + head_off), 0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t dvr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((uint16_t*)a.dv + head_off), 0, head_bytes, kBufferWord3);
  const float sc = a.scale;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * lh;
      const uint32_t off = (uint32_t)(key * KROW + d * 2);
      u32x2 wk, wv;
      wk[0] = E::pack(dka[db][4 * i + 0] * sc, dka[db][4 * i + 1] * sc);
      wk[1] = E::pack(dka[db][4 * i + 2] * sc, dka[db][4 * i + 3] * sc);
      wv[0] = E::pack(dva[db][4 * i + 0], dva[db][4 * i + 1]);
      wv[1] = E::pack(dva[db][4 * i + 2], dva[db][4 * i + 3]);
      __builtin_amdgcn_raw_buffer_store_b64(wk, dkr, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(wv, dvr, off, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV with P handed from one wave of a SIMD to the other: one workgroup per
// (key block of 128 keys, head), 8 waves, two per SIMD; wave w owns keys
// [k_wg + 32*(w%4), +32).  Query tiles of 64 rows (two 32-query sub-blocks),
// copied straight from memory into a 3-stage LDS ring.  Per tile, in two
// phases separated by a barrier:
//   phase 1: the dV wave computes S = Q K_w^T and P = 2^(S c - LSE2) of both
//            sub-blocks and stores the fp32 P in LDS (each lane its own 16
//            values: the dK wave's dP registers have the same layout); the dK
//            wave computes dP = dO V_w^T of both sub-blocks;
//   phase 2: the dV wave accumulates dV^T += dO^T P; the dK wave reads P,
//            forms dS = P (dP - D) and accumulates dK^T += Q^T dS.
// Each product is computed once (8 N^2 d MFMA FLOPs per head) and both waves
// of a SIMD issue 16 MFMAs per phase.
//
// LOOK > 0: the MFMAs of each phase are issued in a fixed order with LOOK
// operand reads ahead (scheduling-group barriers).
template <bool BF16, int D, bool CAUSAL, int LOOK = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fa2_bwd_dkdv_pair_kernel(BwdArgs a) {
  using E = Elem<BF16>;
  constexpr int BK = 128;
  constexpr int SUB = 2;
  constexpr int BQ = 32 * SUB;              // queries per tile
  constexpr int DK = D / 16, DB = D / 32, KROW = D * 2;
  constexpr int TSZ = BQ * KROW;            // bytes of one Q (or dO) tile
  constexpr int STAGE = 2 * TSZ + 2 * 64 * 4;   // Q, dO, 64 LSE slots, 64 D slots
  constexpr int NS = 3;
  constexpr int PSLOT = 64 * 16 * 4;        // one sub-block's fp32 P of one key group (4 KiB)
  constexpr int PBASE = NS * STAGE;
  constexpr int SMEM = PBASE + 4 * SUB * PSLOT;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int grp = wave & 3;                 // key group
  // waves 4-7: dK; waves 0-3: dV (read from lane 0: the role is wave-uniform)
  const bool dk_role = __builtin_amdgcn_readfirstlane(wave) >= 4;

  int bh, kblk;
  {
    const int i = blockIdx.x;
    const int total = a.nblk * a.BH;
    if constexpr (!CAUSAL) {
      const int logical = (total % 8 == 0) ? (i % 8) * (total / 8) + i / 8 : i;
      bh = logical / a.nblk;
      kblk = logical % a.nblk;
    } else {
      bh = i % a.BH;
      kblk = i / a.BH;
    }
  }
  const int N = a.N;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  auto rsrc = [&](const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p + head_off), 0, head_bytes, kBufferWord3);
  };
  const __amdgpu_buffer_rsrc_t qr = rsrc(a.q), kr = rsrc(a.k), vr = rsrc(a.v), dor = rsrc(a.dout);
  const __amdgpu_buffer_rsrc_t lser = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.lse + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t dlr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.delta + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);

  const int k_wg = kblk * BK;
  const int k_w = k_wg + 32 * grp;
  const int key = k_w + lr;

  // the dV wave keeps the group's K rows (for S), the dK wave its V rows (for dP)
  u32x4 bf[DK];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk)
    bf[dk] = __builtin_amdgcn_raw_buffer_load_b128(dk_role ? vr : kr, (uint32_t)(key * KROW + (2 * dk + lh) * 16), 0, 0);
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  const int nt = (N + BQ - 1) / BQ;
  const int t0 = CAUSAL ? k_wg / BQ : 0;

  const FragAddr<D> fa(lane);
  const float c = a.c;
  // this lane's P values of (key group, sub-block): 4 x 16 bytes, lane-contiguous
  uint8_t* const pslot = smem + PBASE + grp * SUB * PSLOT + 16 * lane;

  auto sub_skip = [&](int q0) { return CAUSAL && q0 + 31 < k_w; };   // sub-block entirely before the keys
  auto sub_masked = [&](int q0) { return (q0 + 32 > N) || (CAUSAL && q0 < k_w + 31); };
  // issue order of DK MFMAs fed by one 16-byte read each, LOOK reads ahead
  auto order_fread = [&]() {
    if constexpr (LOOK > 0) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LOOK, 0);
#pragma unroll
      for (int i = 0; i < DK; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (i < DK - LOOK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
    }
  };
  // issue order of 2*DB MFMAs fed by two transpose reads each, LOOK MFMAs ahead
  auto order_tread = [&]() {
    if constexpr (LOOK > 0) {
      constexpr int NM = 2 * DB;
      constexpr int LA = LOOK < NM ? LOOK : NM;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * LA, 0);
#pragma unroll
      for (int i = 0; i < NM - LA; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, LA, 0);
    }
  };

  // phase 1 of one tile: P to LDS (dV wave) or dP into registers (dK wave)
  u32x4 pk[SUB][2];     // dV wave: packed P of each sub-block (B operands of dV^T += dO^T P)
  f32x16 dp[SUB];       // dK wave: dP of each sub-block
  auto phase1 = [&](const uint8_t* st, int t) {
    const uint8_t* qt = st;
    const uint8_t* dot = st + TSZ;
    const float* l2 = (const float*)(st + 2 * TSZ);
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      const int q0 = t * BQ + 32 * sb;
      if (sub_skip(q0)) continue;
      if (!dk_role) {
        f32x16 sv = f32x16{};
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) sv = E::mfma(fa.fread(qt, 32 * sb, dk), bf[dk], sv);
        order_fread();
        const bool masked = sub_masked(q0);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 lq = *(const f32x4*)(l2 + 32 * sb + 8 * g + 4 * lh) * kLog2e;
          f32x4 pv4;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[4 * g + b], c, -lq[b]));
            if (masked) {
              const int q = q0 + 8 * g + 4 * lh + b;
              pv = (q < N && (!CAUSAL || key <= q)) ? pv : 0.f;
            }
            pv4[b] = pv;
          }
          *(f32x4*)(pslot + sb * PSLOT + g * 1024) = pv4;
          pk[sb][g >> 1][2 * (g & 1)] = E::pack(pv4[0], pv4[1]);
          pk[sb][g >> 1][2 * (g & 1) + 1] = E::pack(pv4[2], pv4[3]);
        }
      } else {
        f32x16 d = f32x16{};
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) d = E::mfma(fa.fread(dot, 32 * sb, dk), bf[dk], d);
        order_fread();
        dp[sb] = d;
      }
    }
  };
  // phase 2 of one tile: dV^T += dO^T P (dV wave) or dK^T += Q^T dS (dK wave)
  auto phase2 = [&](const uint8_t* st, int t) {
    const uint8_t* qt = st;
    const uint8_t* dot = st + TSZ;
    const float* dl = (const float*)(st + 2 * TSZ) + 64;
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      const int q0 = t * BQ + 32 * sb;
      if (sub_skip(q0)) continue;
      if (!dk_role) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int h = 0; h < 2; ++h) acc[db] = E::mfma(fa.tread(dot, 32 * sb + 16 * h, db), pk[sb][h], acc[db]);
        order_tread();
      } else {
        u32x4 ds[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 pv4 = *(const f32x4*)(pslot + sb * PSLOT + g * 1024);
          const f32x4 dq4 = *(const f32x4*)(dl + 32 * sb + 8 * g + 4 * lh);
          float v[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) v[b] = pv4[b] * (dp[sb][4 * g + b] - dq4[b]);
          ds[g >> 1][2 * (g & 1)] = E::pack(v[0], v[1]);
          ds[g >> 1][2 * (g & 1) + 1] = E::pack(v[2], v[3]);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int h = 0; h < 2; ++h) acc[db] = E::mfma(fa.tread(qt, 32 * sb + 16 * h, db), ds[h], acc[db]);
      }
    }
  };

  // ---- 3-stage ring of query tiles, two tiles ahead ---------------------------
  // Q, dO, LSE and D go straight from HBM into the ring (buffer_load ... lds
  // issued as inline assembly, no staging registers); each wave waits for its
  // own copies of a tile, then one barrier per tile publishes it and frees the
  // stage of the previous tile.  The compiler does not see the copies (with
  // the builtin it cannot tell the ring's stages apart and drains every copy
  // in flight before each barrier); LSE stays in base e in LDS and is scaled
  // by log2(e) when read.
  constexpr int NI = TSZ / 1024;
  constexpr int IPW = 2 * NI / 8;
  static_assert(2 * NI % 8 == 0 && IPW >= 1 && 2 * (IPW + 1) < 16, "tile copies must split evenly over the waves");
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t dsrc[IPW];
  int ddst[IPW];
  bool dq_t[IPW];
#pragma unroll
  for (int k = 0; k < IPW; ++k) {
    const int i = wv * IPW + k;
    dq_t[k] = i >= NI;
    const int b = (i % NI) * 1024 + 16 * lane;
    const int row = b / KROW, phys = (b % KROW) / 16;
    dsrc[k] = (uint32_t)(row * KROW + 16 * (phys ^ chunk_swizzle<D>(row)));
    ddst[k] = (dq_t[k] ? TSZ : 0) + (i % NI) * 1024;
  }
  const bool stat_wave = wv < 2;            // wave 0: LSE, wave 1: D
  auto dma = [&](int t, int stg) {
    uint8_t* base = smem + stg * STAGE;
    const int qoff = t * BQ * KROW;
#pragma unroll
    for (int k = 0; k < IPW; ++k) lds_dma16_asm(dq_t[k] ? dor : qr, base + ddst[k], dsrc[k], qoff);
    if (stat_wave) lds_dma4_asm(wv == 0 ? lser : dlr, base + 2 * TSZ + (wv == 0 ? 0 : 256), (uint32_t)(4 * lane), t * BQ * 4);
  };
  if (t0 < nt) {
    const int first = nt - t0 < 2 ? nt - t0 : 2;
    for (int i = 0; i < first; ++i) dma(t0 + i, i);
    // the fragment loads are older than every copy: they have landed once at
    // most this wave's copies remain; the empty statements keep the
    // compiler's own wait for them out of the loop
    const int per_tile = IPW + (stat_wave ? 1 : 0);
    if (first * per_tile >= 2 * (IPW + 1)) FA2_WAIT_VMCNT(2 * (IPW + 1));
    else if (first * per_tile >= 2 * IPW) FA2_WAIT_VMCNT(2 * IPW);
    else if (first * per_tile >= IPW + 1) FA2_WAIT_VMCNT(IPW + 1);
    else if (first * per_tile >= IPW) FA2_WAIT_VMCNT(IPW);
    else FA2_WAIT_VMCNT(0);
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) asm volatile("" ::"v"(bf[dk]));
    for (int t = t0; t < nt; ++t) {
      const int i = t - t0;
      // this wave's copies of tile t are done once only tile t+1's may remain
      if (t + 1 < nt) {
        if (stat_wave) FA2_WAIT_VMCNT(IPW + 1);
        else FA2_WAIT_VMCNT(IPW);
      } else {
        FA2_WAIT_VMCNT(0);
      }
      // every wave's copies of tile t have landed and every wave is done with
      // tile t-1 (its stage and the P slots), whose stage now receives tile t+2
      __syncthreads();
      if (t + 2 < nt) dma(t + 2, (i + 2) % 3);
      const uint8_t* st = smem + (i % 3) * STAGE;
      phase1(st, t);
      // the P of both sub-blocks is in LDS
      __syncthreads();
      phase2(st, t);
    }
  }

  // ---- epilogue: dV = dV^T or dK = scale * dK^T, transposed back ----------
  const __amdgpu_buffer_rsrc_t outr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((uint16_t*)(dk_role ? a.dk : a.dv) + head_off), 0, head_bytes, kBufferWord3);
  const float sc = dk_role ? a.scale : 1.f;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * lh;
      u32x2 w;
      w[0] = E::pack(acc[db][4 * i + 0] * sc, acc[db][4 * i + 1] * sc);
      w[1] = E::pack(acc[db][4 * i + 2] * sc, acc[db][4 * i + 3] * sc);
      __builtin_amdgcn_raw_buffer_store_b64(w, outr, (uint32_t)(key * KROW + d * 2), 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV with the P hand-off pipelined across query tiles: the layout of
// fa2_bwd_dkdv_pair_kernel (8 waves, wave w and w+4 own keys
// [k_wg + 32*(w%4), +32), 64-query tiles of two 32-query sub-blocks), with
// one barrier per iteration.  In iteration t:
//   dV wave: dV^T += dO^T P of tile t-1 (P kept packed in registers), then
//            S and P of tile t, P stored packed (16-bit) in LDS slot t % 2;
//   dK wave: P of tile t-1 from slot (t-1) % 2, dS = P (dP - D) with the dP
//            of tile t-1 kept in registers, dK^T += Q^T dS, then dP of tile t.
// Both waves start every iteration with MFMAs that need nothing from the
// other, and each one's VALU work meets the other's MFMAs.  The query tiles
// t-1, t and t+1 are in a 3-stage LDS ring (tile t+1 copied at the start of
// iteration t).  dS is formed from the 16-bit P (its rounding adds at most
// half a unit of the dtype to dS).
template <bool BF16, int D, bool CAUSAL, int LOOK = 4>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fa2_bwd_dkdv_pipe_kernel(BwdArgs a) {
  using E = Elem<BF16>;
  constexpr int BK = 128;
  constexpr int SUB = 2;
  constexpr int BQ = 32 * SUB;
  constexpr int DK = D / 16, DB = D / 32, KROW = D * 2;
  constexpr int TSZ = BQ * KROW;
  constexpr int STAGE = 2 * TSZ + 2 * 64 * 4;
  constexpr int NS = 3;
  constexpr int PSUB = 64 * 32;             // packed P of one sub-block of one key group: 32 bytes per lane
  constexpr int PPAR = SUB * PSUB;          // ... of one tile
  constexpr int PBASE = NS * STAGE;
  constexpr int SMEM = PBASE + 4 * 2 * PPAR;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int grp = wave & 3;
  const bool dk_role = __builtin_amdgcn_readfirstlane(wave) >= 4;

  int bh, kblk;
  {
    const int i = blockIdx.x;
    const int total = a.nblk * a.BH;
    if constexpr (!CAUSAL) {
      const int logical = (total % 8 == 0) ? (i % 8) * (total / 8) + i / 8 : i;
      bh = logical / a.nblk;
      kblk = logical % a.nblk;
    } else {
      bh = i % a.BH;
      kblk = i / a.BH;
    }
  }
  const int N = a.N;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  auto rsrc = [&](const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p + head_off), 0, head_bytes, kBufferWord3);
  };
  const __amdgpu_buffer_rsrc_t qr = rsrc(a.q), kr = rsrc(a.k), vr = rsrc(a.v), dor = rsrc(a.dout);
  const __amdgpu_buffer_rsrc_t lser = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.lse + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t dlr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.delta + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);

  const int k_wg = kblk * BK;
  const int k_w = k_wg + 32 * grp;
  const int key = k_w + lr;

  // the dV wave keeps the group's K rows (for S), the dK wave its V rows (for dP)
  u32x4 bf[DK];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk)
    bf[dk] = __builtin_amdgcn_raw_buffer_load_b128(dk_role ? vr : kr, (uint32_t)(key * KROW + (2 * dk + lh) * 16), 0, 0);
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  const int nt = (N + BQ - 1) / BQ;
  const int t0 = CAUSAL ? k_wg / BQ : 0;

  const FragAddr<D> fa(lane);
  const float c = a.c;
  // this lane's packed P of (key group, parity, sub-block): 2 x 16 bytes, lane-contiguous
  uint8_t* const pslot = smem + PBASE + grp * 2 * PPAR + 16 * lane;

  auto sub_skip = [&](int q0) { return CAUSAL && q0 + 31 < k_w; };
  auto sub_masked = [&](int q0) { return (q0 + 32 > N) || (CAUSAL && q0 < k_w + 31); };
  auto order_fread = [&]() {
    if constexpr (LOOK > 0) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LOOK, 0);
#pragma unroll
      for (int i = 0; i < DK; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (i < DK - LOOK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
    }
  };
  auto order_tread = [&]() {
    if constexpr (LOOK > 0) {
      constexpr int NM = 2 * DB;
      constexpr int LA = LOOK < NM ? LOOK : NM;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * LA, 0);
#pragma unroll
      for (int i = 0; i < NM - LA; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, LA, 0);
    }
  };

  u32x4 pk[SUB][2];     // dV wave: packed P of the previous tile
  f32x16 dp[SUB];       // dK wave: dP of the previous tile
#pragma unroll
  for (int sb = 0; sb < SUB; ++sb) {
    pk[sb][0] = u32x4{};
    pk[sb][1] = u32x4{};
    dp[sb] = f32x16{};
  }

  // tail of tile t (stage st): dV^T += dO^T P (dV wave), or dS and dK^T += Q^T dS (dK wave)
  auto tail = [&](const uint8_t* st, int t) {
    const uint8_t* qt = st;
    const uint8_t* dot = st + TSZ;
    const float* dl = (const float*)(st + 2 * TSZ) + 64;
    const uint8_t* ps = pslot + (t & 1) * PPAR;
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      const int q0 = t * BQ + 32 * sb;
      if (sub_skip(q0)) continue;
      if (!dk_role) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int h = 0; h < 2; ++h) acc[db] = E::mfma(fa.tread(dot, 32 * sb + 16 * h, db), pk[sb][h], acc[db]);
        order_tread();
      } else {
        u32x4 ds[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 pw = *(const u32x4*)(ps + sb * PSUB + h * 1024);
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2) {
            const int r = 8 * h + 2 * t2;          // registers r, r+1: queries of group r/4
            const f32x4 dq4 = *(const f32x4*)(dl + 32 * sb + 8 * (r >> 2) + 4 * lh);
            const float v0 = half_lo<BF16>(pw[t2]) * (dp[sb][r] - dq4[r & 3]);
            const float v1 = half_hi<BF16>(pw[t2]) * (dp[sb][r + 1] - dq4[(r + 1) & 3]);
            ds[h][t2] = E::pack(v0, v1);
          }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int h = 0; h < 2; ++h) acc[db] = E::mfma(fa.tread(qt, 32 * sb + 16 * h, db), ds[h], acc[db]);
      }
    }
  };
  // head of tile t (stage st): S and packed P to registers and LDS (dV wave), or dP (dK wave)
  auto head = [&](const uint8_t* st, int t) {
    const uint8_t* qt = st;
    const uint8_t* dot = st + TSZ;
    const float* l2 = (const float*)(st + 2 * TSZ);
    uint8_t* ps = pslot + (t & 1) * PPAR;
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      const int q0 = t * BQ + 32 * sb;
      if (sub_skip(q0)) continue;
      if (!dk_role) {
        f32x16 sv = f32x16{};
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) sv = E::mfma(fa.fread(qt, 32 * sb, dk), bf[dk], sv);
        order_fread();
        const bool masked = sub_masked(q0);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 lq = *(const f32x4*)(l2 + 32 * sb + 8 * g + 4 * lh) * kLog2e;
          float pv[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[4 * g + b], c, -lq[b]));
            if (masked) {
              const int q = q0 + 8 * g + 4 * lh + b;
              x = (q < N && (!CAUSAL || key <= q)) ? x : 0.f;
            }
            pv[b] = x;
          }
          pk[sb][g >> 1][2 * (g & 1)] = E::pack(pv[0], pv[1]);
          pk[sb][g >> 1][2 * (g & 1) + 1] = E::pack(pv[2], pv[3]);
        }
        *(u32x4*)(ps + sb * PSUB) = pk[sb][0];
        *(u32x4*)(ps + sb * PSUB + 1024) = pk[sb][1];
      } else {
        f32x16 d = f32x16{};
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) d = E::mfma(fa.fread(dot, 32 * sb, dk), bf[dk], d);
        order_fread();
        dp[sb] = d;
      }
    }
  };

  // ---- 3-stage ring: tiles t-1, t, t+1 -----------------------------------------
  constexpr int NI = TSZ / 1024;
  constexpr int IPW = 2 * NI / 8;
  static_assert(2 * NI % 8 == 0 && IPW >= 1 && IPW + 1 < 16, "tile copies must split evenly over the waves");
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t dsrc[IPW];
  int ddst[IPW];
  bool dq_t[IPW];
#pragma unroll
  for (int k = 0; k < IPW; ++k) {
    const int i = wv * IPW + k;
    dq_t[k] = i >= NI;
    const int b = (i % NI) * 1024 + 16 * lane;
    const int row = b / KROW, phys = (b % KROW) / 16;
    dsrc[k] = (uint32_t)(row * KROW + 16 * (phys ^ chunk_swizzle<D>(row)));
    ddst[k] = (dq_t[k] ? TSZ : 0) + (i % NI) * 1024;
  }
  const bool stat_wave = wv < 2;
  auto dma = [&](int t, int stg) {
    uint8_t* base = smem + stg * STAGE;
    const int qoff = t * BQ * KROW;
#pragma unroll
    for (int k = 0; k < IPW; ++k) lds_dma16_asm(dq_t[k] ? dor : qr, base + ddst[k], dsrc[k], qoff);
    if (stat_wave) lds_dma4_asm(wv == 0 ? lser : dlr, base + 2 * TSZ + (wv == 0 ? 0 : 256), (uint32_t)(4 * lane), t * BQ * 4);
  };
  if (t0 < nt) {
    dma(t0, 0);
    // the fragment loads and tile t0 have landed; the empty statements keep
    // the compiler's own wait for the fragments out of the loop
    FA2_WAIT_VMCNT(0);
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) asm volatile("" ::"v"(bf[dk]));
    __syncthreads();
    for (int t = t0; t <= nt; ++t) {
      const int i = t - t0;
      // stage (i+1)%3 held tile t-2, last used in iteration t-1
      if (t + 1 < nt) dma(t + 1, (i + 1) % 3);
      if (t > t0) tail(smem + ((i + 2) % 3) * STAGE, t - 1);
      if (t < nt) head(smem + (i % 3) * STAGE, t);
      // tile t+1 (this iteration's copies) must have landed for iteration t+1
      FA2_WAIT_VMCNT(0);
      __syncthreads();
    }
  }

  // ---- epilogue: dV = dV^T or dK = scale * dK^T, transposed back ----------
  const __amdgpu_buffer_rsrc_t outr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((uint16_t*)(dk_role ? a.dk : a.dv) + head_off), 0, head_bytes, kBufferWord3);
  const float sc = dk_role ? a.scale : 1.f;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * lh;
      u32x2 w;
      w[0] = E::pack(acc[db][4 * i + 0] * sc, acc[db][4 * i + 1] * sc);
      w[1] = E::pack(acc[db][4 * i + 2] * sc, acc[db][4 * i + 3] * sc);
      __builtin_amdgcn_raw_buffer_store_b64(w, outr, (uint32_t)(key * KROW + d * 2), 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (query block of 32*NW queries, head), wave w owns
// queries [q_wg + 32w, +32).  Key tiles of 64 rows: K and V (row-major,
// swizzled) staged in LDS, two stages, register-staged copies one tile
// ahead.
//
// LOOK > 0: the MFMAs of each phase are issued in a fixed order with LOOK
// operand reads ahead (scheduling-group barriers), as in the forward pass.
template <bool BF16, int D, bool CAUSAL, class TL, int LOOK = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(TL::THREADS, TL::THREADS),
                          amdgpu_waves_per_eu(TL::WPE, TL::WPE)))
void fa2_bwd_dq_kernel(BwdArgs a) {
  using E = Elem<BF16>;
  constexpr int T = TL::THREADS, BR = TL::BR, NW = TL::NW;
  constexpr int BC = 64;                    // keys per tile
  constexpr int NKB = BC / 32;
  constexpr int DK = D / 16, DB = D / 32, KROW = D * 2;
  constexpr int TSZ = BC * KROW;
  constexpr int STAGE = 2 * TSZ;
  constexpr int NS = 2;
  constexpr int CH = BC * D / 8;
  constexpr int CH_T = CH / T;
  static_assert(CH % T == 0, "tile copy must split evenly over threads");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;

  int bh, qblk;
  {
    const int i = blockIdx.x;
    const int total = a.nblk * a.BH;
    if constexpr (!CAUSAL) {
      const int logical = (total % 8 == 0) ? (i % 8) * (total / 8) + i / 8 : i;
      bh = logical / a.nblk;
      qblk = logical % a.nblk;
    } else {
      // the last query block sees every key: heaviest first
      bh = i % a.BH;
      qblk = a.nblk - 1 - i / a.BH;
    }
  }
  const int N = a.N;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  auto rsrc = [&](const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)p + head_off), 0, head_bytes, kBufferWord3);
  };
  const __amdgpu_buffer_rsrc_t qr = rsrc(a.q), kr = rsrc(a.k), vr = rsrc(a.v), dor = rsrc(a.dout);

  const int q_wg = qblk * BR;
  const int q_w = q_wg + 32 * wave;
  const int q = q_w + lr;                   // this lane's query (column of S^T, dP^T, dS^T)

  // Q and dO rows of the wave's queries: B operands, kept in VGPRs
  u32x4 qf[DK], dof[DK];
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) {
    const uint32_t off = (uint32_t)(q * KROW + (2 * dk + lh) * 16);
    qf[dk] = __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0);
    dof[dk] = __builtin_amdgcn_raw_buffer_load_b128(dor, off, 0, 0);
  }
  const __amdgpu_buffer_rsrc_t lser = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.lse + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t dlr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.delta + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
  const float lse2 =
      __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lser, (uint32_t)(q * 4), 0, 0)) * kLog2e;
  const float dlt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dlr, (uint32_t)(q * 4), 0, 0));

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  int nt = (N + BC - 1) / BC;
  if constexpr (CAUSAL) {
    const int last_row = min(q_wg + BR, N) - 1;
    nt = min(nt, last_row / BC + 1);
  }

  u32x4 kst[CH_T], vst[CH_T];
  auto load = [&](int key0) {
#pragma unroll
    for (int it = 0; it < CH_T; ++it) {
      const int e = tid + it * T;
      const int row = e / (D / 8), ch = e % (D / 8);
      const uint32_t off = (uint32_t)((key0 + row) * KROW + ch * 16);
      kst[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
      vst[it] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
    }
  };
  auto store = [&](int stg) {
    uint8_t* base = smem + stg * STAGE;
#pragma unroll
    for (int it = 0; it < CH_T; ++it) {
      const int e = tid + it * T;
      const int row = e / (D / 8), ch = e % (D / 8);
      const int off = row * KROW + 16 * (ch ^ chunk_swizzle<D>(row));
      *(u32x4*)(base + off) = kst[it];
      *(u32x4*)(base + TSZ + off) = vst[it];
    }
  };

  const FragAddr<D> fa(lane);
  const float c = a.c;

  auto compute = [&](const uint8_t* st, int key0, bool masked) {
    const uint8_t* kt = st;
    const uint8_t* vt = st + TSZ;
    // S^T = K Q_w^T, dP^T = V dO_w^T: keys as rows, the wave's queries as columns
    f32x16 s[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
    }
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = E::mfma(fa.fread(kt, 32 * kb, dk), qf[dk], s[kb]);
        dp[kb] = E::mfma(fa.fread(vt, 32 * kb, dk), dof[dk], dp[kb]);
      }
    }
    if constexpr (LOOK > 0) {
      // one 16-byte operand read per MFMA, LOOK reads ahead
      constexpr int NM = 2 * NKB * DK;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LOOK, 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (i < NM - LOOK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
    }
    // P^T = 2^(s*c - LSE2), dS^T = P^T * (dP^T - D), packed (registers
    // [8h, 8h+8) = 16-key step h)
    u32x4 dsp[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -lse2));
        if (masked) {
          const int kk = key0 + 32 * kb + 8 * (r >> 2) + 4 * lh + (r & 3);
          const bool vis = kk < N && (!CAUSAL || kk <= q);
          pv = vis ? pv : 0.f;
        }
        ds[r] = pv * (dp[kb][r] - dlt);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) dsp[kb][h][t] = E::pack(ds[8 * h + 2 * t], ds[8 * h + 2 * t + 1]);
    }
    // dQ^T += K^T dS^T (k = 16 renumbered keys per step)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[db] = E::mfma(fa.tread(kt, 32 * kb + 16 * h, db), dsp[kb][h], acc[db]);
    if constexpr (LOOK > 0) {
      // two transpose reads per MFMA, 2*LOOK reads ahead
      constexpr int NM = DB * NKB * 2;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * LOOK, 0);
#pragma unroll
      for (int i = 0; i < NM - LOOK; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, LOOK, 0);
    }
  };

  auto tile = [&](const uint8_t* st, int j) {
    const int key0 = j * BC;
    const bool skip = CAUSAL && key0 > q_w + 31;   // tile entirely above this wave's diagonal
    if (!skip) {
      const bool masked = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q_w);
      compute(st, key0, masked);
    }
  };

  load(0);
  store(0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  for (int j = 0; j < nt; ++j) {
    if (j + 1 < nt) load((j + 1) * BC);
    tile(smem + (j & 1) * STAGE, j);
    if (j + 1 < nt) store((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: dQ = scale * dQ^T (transposed back) ----------------------
  const __amdgpu_buffer_rsrc_t dqr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((uint16_t*)a.dq + head_off), 0, head_bytes, kBufferWord3);
  const float sc = a.scale;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * lh;
      u32x2 w;
      w[0] = E::pack(acc[db][4 * i + 0] * sc, acc[db][4 * i + 1] * sc);
      w[1] = E::pack(acc[db][4 * i + 2] * sc, acc[db][4 * i + 3] * sc);
      __builtin_amdgcn_raw_buffer_store_b64(w, dqr, (uint32_t)(q * KROW + d * 2), 0, 0);
    }
  }
}

}  // namespace fa2
