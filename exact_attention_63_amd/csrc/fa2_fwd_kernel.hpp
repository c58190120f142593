// fa2_fwd_kernel.hpp -- exact attention forward for gfx950 (CDNA4): one
// workgroup per (query block, head, batch), sliced-Q over 64-lane waves,
// online softmax in registers, both products on MFMA.
//
// Method: "FlashAttention v2 better parallelism + work partitioning" diagram.
//   * grid over (batch, head, query block): the "parallel for batch, head,
//     q_block" loop of the concept pseudo-code panel and the sequence-length
//     parallelism of the "what v2 changes" panel;
//   * the rows of a query block are split across the waves of the workgroup,
//     each wave keeps its own (m, l, acc) and writes its own output rows, and
//     the K/V tile is loaded once into shared memory for all waves (sliced-Q
//     panel and the thread/data-movement panel);
//   * per key tile: S = Q K^T, mask only where a mask can matter, online
//     softmax update, acc += P V (concept pseudo-code panel);
//   * final O = acc / l once at the end ("FlashAttention v4 Blackwell pipeline
//     co-design" diagram, pseudo-code panel), so no per-tile divide.
//
// MI355X-specific design (none of this is on the pages, which target NVIDIA):
//   * Scores are produced transposed, S^T = K Q^T, with the 32x32x16 MFMA.  In
//     that layout a lane holds one query (lane % 32) and 16 keys per 32x32
//     block, so the row max, the row sum and the rescale of acc by alpha are
//     in-lane; only one exchange between lane l and lane l^32
//     (v_permlane32_swap) is needed per row statistic.  The output is accumulated transposed too,
//     O^T += V^T P^T, whose B operand (keys x queries) is exactly the S^T
//     accumulator registers [8s, 8s+8) of each 16-key step s once keys are
//     renumbered inside every 32-key block (slot 16s+8h+4a+b holds key
//     16s+8a+4h+b).  P therefore never leaves registers.
//   * K and V are both staged row-major [key][d].  K fragments are 16-byte
//     LDS reads; V^T fragments (keys along the MFMA k dimension) come from
//     the gfx950 LDS transpose read ds_read_b64_tr_b16, whose lane mapping
//     also realises the key renumbering above, so V needs no transpose in
//     registers.
//   * The default loops copy K and V tiles straight from HBM into a ring of
//     LDS stages (buffer_load ... lds), unpadded, with the 16-byte chunks of
//     each row XOR-swizzled (chunk_swizzle) so that the lanes one LDS cycle
//     serves fall on distinct banks of the 64 x 4-byte bank array -- the
//     bank-conflict fix of blog chapter 4.  The older register-staged loops
//     pad the rows instead (K pitch 16 mod 256 bytes, V pitch 64 mod 256).
//   * Global reads and writes use buffer instructions with the head's extent
//     as the range: rows past N read as zero and their stores are dropped, so
//     ragged N needs no branches in the copy code.
//   * Scale is folded into one FMA feeding exp2: p = 2^(s*c - m) with
//     c = scale*log2(e) (blog chapter 6, FP instruction fusion); m, l are
//     kept in the base-2 domain; LSE = (m + log2 l) * ln 2 at the end.  A
//     negative scale flips the sign of Q once, so c >= 0 in every loop.
//   * The reference max of a row moves only when a tile's max exceeds it by
//     more than kLazyRescale (the conditional rescale of the v4 diagram, in
//     an exact form), so acc is rescaled only in the rare tiles where it
//     moves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>


namespace fa2 {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Buffer descriptor word 3 for raw (untyped) buffer access on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;
// Lazy rescale threshold in base-2 units: p never exceeds 2^8 = 256.
constexpr float kLazyRescale = 8.f;
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;
// VALU instructions placed after each score MFMA in the interleaved loop.
constexpr int kValuPerMfma = 8;

template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> packed pair, round to nearest even (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

template <>
struct Elem<false> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// Combine a per-lane value with the one held 32 lanes away, leaving the
// result in both lanes.  v_permlane32_swap(x, x) returns {x of lanes 0-31 in
// both halves, x of lanes 32-63 in both halves}: one VALU op, no LDS.
__device__ __forceinline__ float max_halves(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
}

// XOR swizzle of the 16-byte chunks of an unpadded LDS row of D 16-bit
// elements (D = 128: 16 chunks, D = 64: 8 chunks).  With it, the 16 rows read
// at one chunk by a 16-byte fragment read, and the 4 rows x 64 bytes of one
// transpose read, fall on distinct banks of the 64 x 4-byte bank array.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    static_assert(D == 64, "d must be 64 or 128");
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
}

// 16 bytes per lane from a buffer straight into LDS: lane l of the wave writes
// lds + 16*l (buffer_load_dwordx4 ... lds; out-of-range lanes write zeros).
// Kept in a device-only function: used directly in the kernel body, the
// builtin makes the host compilation pass drop the kernel's launch stub.
// With the builtin the compiler tracks the copy as an LDS write and makes
// later LDS reads that it cannot tell apart from the destination (the
// transpose reads) wait for every copy in flight.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voffset,
                                          int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds), 16, voffset,
                                           soffset, 0, 0);
}
// The same copy as inline assembly (Tile::ASMDMA): the compiler then does not
// track it at all, and the kernel's own ordering is the only one: each wave
// waits for its copies of a stage with s_waitcnt vmcnt, then a barrier
// publishes the stage.  M0 holds the LDS destination; one wait state
// separates its write from the copy.
__device__ __forceinline__ void lds_dma16_asm(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voffset,
                                              int soffset) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(dst), "v"(voffset), "s"(r), "s"(soffset)
               : "memory", "m0");
}

// 2^x on the FMA pipe instead of the transcendental unit: the software exp2
// of the "FlashAttention v4 Blackwell pipeline co-design" diagram, kept here
// as a measured alternative (Tile::SWEXP).  x = n + f with n = floor(x) and
// f in [0, 1); 2^f from a degree-4 polynomial fitted to the relative error on
// [0, 1] (gen_exp2_poly.py: at most 2.9e-6, far below the 2^-9 rounding of P
// to bf16); 2^n applied with ldexp.  Arguments below -126 (masked scores are
// -inf) give exactly 0.  The softmax arguments never exceed 8.
__device__ __forceinline__ float sw_exp2(float x) {
  const float xc = fmaxf(x, -127.f);
  const float n = __builtin_floorf(xc);
  const float f = xc - n;
  float p = __builtin_fmaf(0.013426551595330238f, f, 0.052240896970033646f);
  p = __builtin_fmaf(p, f, 0.24128268659114838f);
  p = __builtin_fmaf(p, f, 0.6930440068244934f);
  p = __builtin_fmaf(p, f, 1.0f);
  const float r = __builtin_ldexpf(p, (int)n);
  return x < -126.f ? 0.f : r;
}

// s_waitcnt vmcnt(n) (n < 16) with expcnt and lgkmcnt left at their maxima.
#define FA2_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))

// Calls f(integral_constant<I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// The two MFMA phases of a 64-key tile as inline-assembly blocks with a
// fixed LDS-operand lookahead (generated by gen_mfma_phases.py).
#include "fa2_mfma_phases.inc"

// ds_read_b64_tr_b16: transpose read of 16-bit elements (see the V fragment
// comment in the kernel for the lane mapping).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

struct Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;      // B*H
  int N;       // sequence length
  int nqb;     // query blocks per head
  float c;     // scale * log2(e)
};

// Tile configuration.
//   NW : waves per workgroup         QB : 32-query blocks per wave
//   KB : 32-key blocks per key tile  WPE: waves per SIMD the kernel is built for
//   PIPE: software-pipelined main loop (see below)
template <int NW_, int QB_, int KB_, int WPE_, int PIPE_ = 0, int LOOK_ = 0, int PRE_ = 0,
          bool ASMDMA_ = false, int ASMPH_ = 0, int SWEXP_ = 0>
struct Tile {
  static constexpr int NW = NW_, QB = QB_, KB = KB_, WPE = WPE_;
  // SWEXP: the softmax's 2^x from sw_exp2 (FMA pipe) for every score (1), for
  // every other score (2), or from v_exp_f32 only (0)
  static constexpr int SWEXP = SWEXP_;
  // ASMPH (direct-copy loops, d = 128, 32 rows per wave, 64-key tiles):
  // issue each MFMA phase of a tile (16 score MFMAs; 16 P.V MFMAs) as one
  // inline-assembly block that keeps ASMPH MFMAs' worth of LDS operand
  // reads in flight and waits with exact counts (0: compiler-scheduled)
  static constexpr int ASMPH = ASMPH_;
  // ASMDMA (direct-copy loops): issue the global->LDS copies as inline
  // assembly, invisible to the compiler's wait-count tracking
  static constexpr bool ASMDMA = ASMDMA_;
  // PRE (direct-copy loops): PIPE 4/5/7: number of P.V operands (V^T
  // fragments) read from LDS before the softmax, so that the P.V MFMAs can
  // start without waiting; PIPE 9: the same operands read during the softmax
  // half-step; PIPE 10: MFMA operands read ahead in the threaded region
  // (0 means 4)
  static constexpr int PRE = PRE_;
  // LOOK (direct-copy loops): keep this many score-MFMA operand reads in
  // flight ahead of the MFMAs (0: leave the order to the compiler)
  static constexpr int LOOK = LOOK_;
  // PIPE 1: issue the next tile's score MFMAs in the same basic block as the
  // current tile's softmax (K staged two tiles ahead, V one tile ahead);
  // PIPE 2: additionally ask the scheduler to interleave those MFMAs with the
  // softmax VALU work one by one, so that one wave keeps both pipes busy;
  // PIPE 3: ping-pong between two wave groups in opposite phases;
  // PIPE 4 / 5: K and V copied straight from HBM into a 3- / 2-stage LDS ring
  // (buffer_load ... lds), swizzled unpadded rows;
  // PIPE 7: 4-stage ring with one barrier per two tiles;
  // PIPE 9: 4-stage ring, two wave groups in opposite phases (ping-pong);
  // PIPE 10: 4-stage ring, 32-key blocks, each wave's softmax threaded
  // between its own MFMAs (see the loop);
  // PIPE 11: 3-stage ring, waves 0-3 run one phase ahead of waves 4-7.
  static constexpr int PIPE = PIPE_;
  static constexpr int BR = NW * 32 * QB;  // query rows per workgroup
  static constexpr int BC = 32 * KB;       // keys per tile
  static constexpr int THREADS = NW * 64;
};

template <bool BF16, int D, bool CAUSAL, class TL>
__global__ __attribute__((amdgpu_flat_work_group_size(TL::THREADS, TL::THREADS),
                          amdgpu_waves_per_eu(TL::WPE, TL::WPE)))
void fa2_fwd_kernel(Args a) {
  using E = Elem<BF16>;
  constexpr int NW = TL::NW, QB = TL::QB, KB = TL::KB;
  constexpr int BR = TL::BR, BC = TL::BC, T = TL::THREADS;
  constexpr int DK = D / 16;            // 16-wide k steps of the score product
  constexpr int DB = D / 32;            // 32-row blocks of O^T
  constexpr int KROW = D * 2;           // bytes per K (and Q, V, O) row in HBM
  constexpr int KP = KROW + 16;         // K row pitch in LDS (16 mod 128: 16-byte reads of 8 rows)
  constexpr int VP = KROW + 64;         // V row pitch in LDS (64 mod 256: 64-byte runs of 4 rows)
  constexpr int KSTAGE = BC * KP;       // bytes of one K tile
  constexpr int VSTAGE = BC * VP;       // bytes of one V tile
  constexpr int STAGE = KSTAGE + VSTAGE;  // LDS: K stage 0, K stage 1, V stage 0, V stage 1
  constexpr int CH = BC * D / 8;        // 16-byte chunks per K (or V) tile
  constexpr int CH_T = CH / T;          // ... per thread
  static_assert(CH % T == 0, "tile copy must split evenly over threads");
  // PIPE 4 (direct global->LDS copies): 3 stages of unpadded, XOR-swizzled
  // [key][d] K and V tiles
  constexpr int TSZ = BC * KROW;        // bytes of one unpadded K (or V) tile
  // LDS stages of the direct-copy loops (PIPE 4 and 11: 3, PIPE 5: 2, PIPE 7, 9 and 10: 4)
  constexpr int NS = (TL::PIPE == 4 || TL::PIPE == 11) ? 3 : ((TL::PIPE == 7 || TL::PIPE == 9 || TL::PIPE == 10) ? 4 : 2);
  constexpr bool DMA = TL::PIPE == 4 || TL::PIPE == 5 || TL::PIPE == 7 || TL::PIPE == 9 || TL::PIPE == 10 ||
                       TL::PIPE == 11;
  constexpr int SMEM = DMA ? NS * 2 * TSZ : 2 * STAGE;
  // hand-scheduled MFMA phases exist for d = 128, 32 rows per wave, 64-key tiles
  constexpr int ASMPH = (DMA && D == 128 && QB == 1 && KB == 2) ? TL::ASMPH : 0;
  static_assert(SMEM <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;   // query (S^T column) / row index inside a 32-block
  const int lh = lane >> 5;   // which half of the 64-lane wave

  // ---- workgroup -> (query block, head) --------------------------------
  // Non-causal: all workgroups do equal work; consecutive logical ids walk the
  // query blocks of one head and are kept on one XCD (workgroups are dealt to
  // the 8 XCDs round-robin), so a head's K/V stay in that XCD's L2.
  // Causal: heaviest query blocks first; with B*H a multiple of 8 each XCD
  // then owns a fixed set of heads.
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
  const size_t head_off = (size_t)bh * (size_t)N * D;   // elements
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.q + head_off), 0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.k + head_off), 0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.v + head_off), 0, head_bytes, kBufferWord3);

  const int q_wg = qblk * BR;                 // first query row of the workgroup
  const int q_w = q_wg + wave * 32 * QB;      // first query row of this wave

  // number of key tiles this workgroup visits
  int nt = (N + BC - 1) / BC;
  if constexpr (CAUSAL) {
    const int last_row = min(q_wg + BR, N) - 1;
    nt = min(nt, last_row / BC + 1);
  }

  // ---- Q fragments (B operand of S^T = K Q^T), kept in VGPRs -------------
  u32x4 qf[QB][DK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q_w + qb * 32 + lr;
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      qf[qb][dk] = __builtin_amdgcn_raw_buffer_load_b128(qr, (uint32_t)(row * KROW + (2 * dk + lh) * 16), 0, 0);
    }
  }

  // ---- staging registers for the next K/V tile ---------------------------
  // Thread tid copies 16-byte chunks tid, tid + T, ... of each tile; a row of
  // d elements is d/8 consecutive chunks, so a wave reads whole rows.
  u32x4 kst[CH_T], vst[CH_T];
  uint8_t* const kring = smem;                 // K stages 0, 1
  uint8_t* const vring = smem + 2 * KSTAGE;    // V stages 0, 1

  auto load_k = [&](int key0) {
#pragma unroll
    for (int it = 0; it < CH_T; ++it) {
      const int e = tid + it * T;
      const int row = e / (D / 8), ch = e % (D / 8);
      kst[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, (uint32_t)((key0 + row) * KROW + ch * 16), 0, 0);
    }
  };
  auto load_v = [&](int key0) {
#pragma unroll
    for (int it = 0; it < CH_T; ++it) {
      const int e = tid + it * T;
      const int row = e / (D / 8), ch = e % (D / 8);
      vst[it] = __builtin_amdgcn_raw_buffer_load_b128(vr, (uint32_t)((key0 + row) * KROW + ch * 16), 0, 0);
    }
  };
  auto store_k = [&](int stage) {
#pragma unroll
    for (int it = 0; it < CH_T; ++it) {
      const int e = tid + it * T;
      const int row = e / (D / 8), ch = e % (D / 8);
      *(u32x4*)(kring + stage * KSTAGE + row * KP + ch * 16) = kst[it];
    }
  };
  auto store_v = [&](int stage) {
#pragma unroll
    for (int it = 0; it < CH_T; ++it) {
      const int e = tid + it * T;
      const int row = e / (D / 8), ch = e % (D / 8);
      *(u32x4*)(vring + stage * VSTAGE + row * VP + ch * 16) = vst[it];
    }
  };

  // ---- per-row online-softmax state (base-2 domain) ----------------------
  f32x16 acc[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
  }
  // A negative scale is folded into Q: c*s = (-c)*(-s) exactly (negating a
  // 16-bit float flips its sign bit), so every loop below sees c >= 0, and
  // the row max of c*s is c times the row max of s.
  const bool c_neg = a.c < 0.f;
  const float c = c_neg ? -a.c : a.c;
  if (c_neg) {
    const u32x4 sign = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) qf[qb][dk] ^= sign;
  }
  const int kbase = lr * KP + lh * 16;   // this lane's K fragment: row 32*kb + lr, chunk 2*dk + lh
  // V^T fragments come from row-major V through the LDS transpose read.  In
  // each 16-lane group g, lane (4e + c) fetches 4 elements of key row
  // 4*(g/2) + e at columns 16*(g%2) + 4c; the hardware hands lane i of the
  // group element i of each of the group's 4 rows, which is the A operand
  // layout (d = lane % 32, keys 4*(lane/32) + 0..3 of the renumbered step).
  const int vg = lane >> 4;
  const int vbase = (4 * (vg >> 1) + ((lane >> 2) & 3)) * VP + 32 * (vg & 1) + 8 * (lane & 3);

  // S^T = K Q^T for every (key block, query block), K from one LDS stage
  auto scores = [&](const uint8_t* ks, f32x16 (&s)[QB][KB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4 kf = *(const u32x4*)(ks + kbase + 32 * kb * KP + 32 * dk);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = E::mfma(kf, qf[qb][dk], s[qb][kb]);
      }
    }
  };

  // online softmax of one tile of scores: updates m, l, returns P and alpha
  // s: f32x16[QB][NBK] scores of NBK 32-key blocks starting at key0,
  // pf: u32x4[QB][NBK][2] packed P
  auto softmax = [&](auto& s, int key0, bool masked, auto& pf, float (&alpha)[QB]) __attribute__((always_inline)) {
    constexpr int NBK = sizeof(s[0]) / sizeof(f32x16);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float cc = c;
      float m_tile;
      if (masked) {
        // tiles that cross the diagonal or the end of the sequence: scale
        // first, masked scores become -inf and exp2 gives exactly 0 for them
        const int q = q_w + qb * 32 + lr;
        float e0 = -INFINITY, e1 = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * lh + (r & 3);
            const bool vis = key < N && (!CAUSAL || key <= q);
            const float t = vis ? s[qb][kb][r] * c : -INFINITY;
            s[qb][kb][r] = t;
            if (r & 1) e1 = fmaxf(e1, t); else e0 = fmaxf(e0, t);
          }
        m_tile = max_halves(fmaxf(e0, e1));
        cc = 1.f;
      } else {
        // c >= 0 here, so the tile max of c*s is c*max(s); two chains
        float e0 = s[qb][0][0], e1 = s[qb][0][1];
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            e0 = fmaxf(e0, fmaxf(s[qb][kb][r], s[qb][kb][r + 1]));
            e1 = fmaxf(e1, fmaxf(s[qb][kb][r + 2], s[qb][kb][r + 3]));
          }
        m_tile = max_halves(fmaxf(e0, e1)) * c;
      }
      // Lazy reference: the row's reference max moves only when the tile max
      // exceeds it by more than kLazyRescale (or it is still -inf); otherwise
      // alpha = 1 and p = 2^(s*c - m) stays below 2^kLazyRescale.  O = acc / l
      // and LSE = m + log2 l use the same reference, so the result is the same
      // exact value (the conditional rescale of the v4 diagram, exact form).
      const float m_old = m_run[qb];
      const float m_new = (m_tile > m_old + kLazyRescale) ? m_tile : m_old;
      // a row with no visible key so far keeps m = -inf; never form -inf - -inf
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      alpha[qb] = __builtin_amdgcn_exp2f(m_old - m_use);
      m_run[qb] = m_new;
      // p = 2^(s*c - m): one FMA + one exp2 per score.  The row sum is taken
      // over the fp32 p (two chains): summing the 16-bit P instead would put
      // its rounding (2^-9 relative in bf16) straight into LSE.  P is rounded
      // to the input type for the P.V product.
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < NBK; ++kb) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float p[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float x = __builtin_fmaf(s[qb][kb][8 * st + t], cc, -m_use);
            if constexpr (TL::SWEXP == 1) {
              p[t] = sw_exp2(x);
            } else if constexpr (TL::SWEXP == 2) {
              p[t] = (t & 1) ? sw_exp2(x) : __builtin_amdgcn_exp2f(x);
            } else {
              p[t] = __builtin_amdgcn_exp2f(x);
            }
            if (t & 1) rs1 += p[t]; else rs0 += p[t];
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) pf[qb][kb][st][t] = E::pack(p[2 * t], p[2 * t + 1]);
        }
      }
      l_run[qb] = l_run[qb] * alpha[qb] + (rs0 + rs1);
    }
  };

  // acc = alpha * acc (only when some row moved its reference), then
  // O^T += V^T P^T with V from one LDS stage
  auto rescale_pv = [&](const uint8_t* vs, const u32x4 (&pf)[QB][KB][2], const float (&alpha)[QB]) {
    // rescale acc only when some row of the wave moved its reference
    bool moved = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) moved |= alpha[qb] != 1.f;
    if (__any(moved)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha[qb];
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint8_t* vp = vs + vbase + (32 * kb + 16 * st) * VP + 64 * db;
          const u32x2 lo = lds_read_tr16(vp);            // keys 4h + 0..3 of the step
          const u32x2 hi = lds_read_tr16(vp + 8 * VP);   // keys 8 + 4h + 0..3
          const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][db] = E::mfma(vf, pf[qb][kb][st], acc[qb][db]);
        }
      }
    }
  };

  auto tile_skip = [&](int key0) {     // tile entirely above this wave's diagonal
    return CAUSAL && key0 > q_w + 32 * QB - 1;
  };
  auto tile_masked = [&](int key0) {   // tile crosses the diagonal or the end of the sequence
    return (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q_w);
  };

  if constexpr (TL::PIPE == 0) {
    // ---- main loop: 2-stage LDS ring, next tile's loads overlap compute ----
    load_k(0);
    load_v(0);
    store_k(0);
    store_v(0);
    // Every load issued so far (Q fragments, first tile) is complete here.
    // Saying so explicitly keeps the compiler from placing waits for the Q
    // loads inside the loop, where they would also wait for the prefetch of
    // the next tile and expose its latency on every iteration.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
      const int key0 = j * BC;
      if (j + 1 < nt) {
        load_k(key0 + BC);
        load_v(key0 + BC);
      }
      if (!tile_skip(key0)) {
        f32x16 sc[QB][KB];
        u32x4 pf[QB][KB][2];
        float alpha[QB];
        scores(kring + (j & 1) * KSTAGE, sc);
        softmax(sc, key0, tile_masked(key0), pf, alpha);
        rescale_pv(vring + (j & 1) * VSTAGE, pf, alpha);
      }
      if (j + 1 < nt) {
        store_k((j + 1) & 1);
        store_v((j + 1) & 1);
      }
      __syncthreads();
    }
  } else if constexpr (DMA) {
    // ---- direct global->LDS copies, NS-stage ring ---------------------------
    // Each K/V tile is fetched NS-1 tiles ahead with buffer_load ... lds: the
    // data never passes through VGPRs, and every wave only waits for its own
    // copies of the tile it is about to use.  One DMA instruction writes 1 KiB
    // of LDS, lane l at byte 16*l, so the bank-conflict fix is an XOR swizzle
    // of 16-byte chunks inside each row (chunk_swizzle) applied through the
    // choice of source address; the fragment reads apply the same swizzle.
    // LDS: K stage s at s*TSZ, V stage s at (NS + s)*TSZ.  The loop is
    // unrolled by the NS stages so that every LDS offset is an immediate on a
    // handful of per-lane base registers.
    constexpr int NI = TSZ / 1024;     // DMA instructions per tile and tensor
    static_assert(NI % NW == 0, "tile DMA must split evenly over the waves");
    constexpr int NIW = NI / NW;       // ... per wave
    // per-lane source offsets of this wave's DMA instructions (row, logical chunk)
    uint32_t dsrc[NIW];
#pragma unroll
    for (int k = 0; k < NIW; ++k) {
      const int b = (wave * NIW + k) * 1024 + 16 * lane;
      const int row = b / KROW, phys = (b % KROW) / 16;
      dsrc[k] = (uint32_t)(row * KROW + 16 * (phys ^ chunk_swizzle<D>(row)));
    }
    auto dma = [&](int tile, auto stage_tag) {
      constexpr int S = decltype(stage_tag)::value;
      const int base = tile * BC * KROW;      // uniform: the SGPR offset of the copy
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        const int dst = (wave * NIW + k) * 1024;
        if constexpr (TL::ASMDMA) {
          lds_dma16_asm(kr, smem + S * TSZ + dst, dsrc[k], base);
          lds_dma16_asm(vr, smem + (NS + S) * TSZ + dst, dsrc[k], base);
        } else {
          lds_dma16(kr, smem + S * TSZ + dst, dsrc[k], base);
          lds_dma16(vr, smem + (NS + S) * TSZ + dst, dsrc[k], base);
        }
      }
    };
    // The compiler does not count the copies (assembly) or does not relate
    // them to Q, so it may believe the Q loads are still in flight inside the
    // loop and wait for them (and so for every copy issued after them) there.
    // Once the explicit wait has covered Q, pass the Q registers through an
    // empty statement: the compiler's own wait for them lands here, before
    // the loop.
    auto q_ready = [&]() {
      static_assert(QB * DK <= 16, "Q fragment count");
      const u32x4* qq = &qf[0][0];
      if constexpr (QB * DK == 4) {
        asm volatile("" ::"v"(qq[0]), "v"(qq[1]), "v"(qq[2]), "v"(qq[3]));
      } else if constexpr (QB * DK == 8) {
        asm volatile("" ::"v"(qq[0]), "v"(qq[1]), "v"(qq[2]), "v"(qq[3]), "v"(qq[4]), "v"(qq[5]), "v"(qq[6]),
                     "v"(qq[7]));
      } else {
        asm volatile("" ::"v"(qq[0]), "v"(qq[1]), "v"(qq[2]), "v"(qq[3]), "v"(qq[4]), "v"(qq[5]), "v"(qq[6]),
                     "v"(qq[7]), "v"(qq[8]), "v"(qq[9]), "v"(qq[10]), "v"(qq[11]), "v"(qq[12]), "v"(qq[13]),
                     "v"(qq[14]), "v"(qq[15]));
      }
    };
    // fragment addresses (see chunk_swizzle): K row 32*kb + lr, chunk 2*dk + lh;
    // V rows 32*kb + 16*st + 8*x + 4*(g/2) + e, chunk 4*db + 2*(g%2) + c/2
    const int kfb = lr * KROW + 16 * (lh ^ chunk_swizzle<D>(lr));
    const int vgq = lane >> 4, ve = (lane >> 2) & 3, vc = lane & 3;
    const int vfb = (4 * (vgq >> 1) + ve) * KROW + 8 * (vc & 1) +
                    (D == 128 ? 64 * ve : 64 * (ve >> 1)) +
                    16 * ((2 * (vgq & 1) | (vc >> 1)) ^ (vgq >> 1));
    int ka[DK];                 // K fragment base of each 16-wide d step
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) ka[dk] = kfb ^ (32 * dk);
    int va[DB][2];              // V fragment base of each 32-wide d block, low/high 8 keys
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      va[db][0] = NS * TSZ + (vfb ^ (64 * db));
      va[db][1] = NS * TSZ + 8 * KROW + (vfb ^ (64 * db) ^ 32);
    }
    // S^T = K Q^T from K stage S
    // LDS byte address of smem (the kernel's only LDS allocation)
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    auto scores_st = [&](f32x16 (&sv)[QB][KB], auto stage_tag) {
      constexpr int S = decltype(stage_tag)::value;
      if constexpr (ASMPH > 0) {
        const uint32_t k0 = lds0 + ka[0], k1 = lds0 + ka[1], k2 = lds0 + ka[2], k3 = lds0 + ka[3];
        const uint32_t k4 = lds0 + ka[4], k5 = lds0 + ka[5], k6 = lds0 + ka[6], k7 = lds0 + ka[7];
#define FA2_SCORES_OPERANDS                                                                                   \
  : [s0] "=&v"(sv[0][0]), [s1] "=&v"(sv[0][1])                                                               \
  : [ka0] "v"(k0), [ka1] "v"(k1), [ka2] "v"(k2), [ka3] "v"(k3), [ka4] "v"(k4), [ka5] "v"(k5), [ka6] "v"(k6), \
    [ka7] "v"(k7), [q0] "v"(qf[0][0]), [q1] "v"(qf[0][1]), [q2] "v"(qf[0][2]), [q3] "v"(qf[0][3]),          \
    [q4] "v"(qf[0][4]), [q5] "v"(qf[0][5]), [q6] "v"(qf[0][6]), [q7] "v"(qf[0][7]), [o0] "n"(S * TSZ),      \
    [o1] "n"(S * TSZ + 32 * KROW)
        if constexpr (BF16) {
          static_assert(ASMPH == 4 || ASMPH == 8, "generated lookaheads: 4, 8");
          if constexpr (ASMPH == 4) asm volatile(FA2_ASM_SCORES_BF16_L4 FA2_SCORES_OPERANDS : "memory", FA2_ASM_CLOBBERS_L4);
          else asm volatile(FA2_ASM_SCORES_BF16_L8 FA2_SCORES_OPERANDS : "memory", FA2_ASM_CLOBBERS_L8);
        } else {
          static_assert(ASMPH == 4 || ASMPH == 8, "generated lookaheads: 4, 8");
          if constexpr (ASMPH == 4) asm volatile(FA2_ASM_SCORES_F16_L4 FA2_SCORES_OPERANDS : "memory", FA2_ASM_CLOBBERS_L4);
          else asm volatile(FA2_ASM_SCORES_F16_L8 FA2_SCORES_OPERANDS : "memory", FA2_ASM_CLOBBERS_L8);
        }
#undef FA2_SCORES_OPERANDS
        return;
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sv[qb][kb] = f32x16{};
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const u32x4 kf = *(const u32x4*)(smem + ka[dk] + (S * TSZ + 32 * kb * KROW));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sv[qb][kb] = E::mfma(kf, qf[qb][dk], sv[qb][kb]);
        }
      }
    };
    // issue order for a score product: LOOK fragment reads ahead, then one
    // MFMA per further read, with VALU instructions of the same basic block
    // (VPM per MFMA) filling the MFMA shadow
    auto order_scores = [&](auto look_tag, auto vpm_tag) {
      constexpr int LOOK = decltype(look_tag)::value, VPM = decltype(vpm_tag)::value;
      constexpr int NM = QB * KB * DK, NR = KB * DK;
      static_assert(QB == 1, "read lookahead assumes one fragment per MFMA");
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LOOK, 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (i < NR - LOOK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        if constexpr (VPM > 0) __builtin_amdgcn_sched_group_barrier(kSchedValu, VPM, 0);
      }
    };
    // V^T operand of the P.V MFMA for (32-wide d block db, key block kb,
    // 16-key step st) from V stage S
    auto vread = [&](int db, int kb, int st, auto stage_tag) {
      constexpr int S = decltype(stage_tag)::value;
      const int roff = S * TSZ + (32 * kb + 16 * st) * KROW;
      const u32x2 lo = lds_read_tr16(smem + va[db][0] + roff);   // keys 4h + 0..3 of the step
      const u32x2 hi = lds_read_tr16(smem + va[db][1] + roff);   // keys 8 + 4h + 0..3
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    constexpr int NPV = DB * KB * 2;            // P.V MFMAs per query block
    constexpr int NPRE = TL::PRE < NPV ? TL::PRE : NPV;
    typedef u32x4 PreOps[NPRE > 0 ? NPRE : 1];
    // the first NPRE operands, in P.V order (db outer, then kb, then st)
    auto vpre = [&](PreOps& pre, auto stage_tag) {
#pragma unroll
      for (int i = 0; i < NPRE; ++i) pre[i] = vread(i / (KB * 2), (i / 2) % KB, i % 2, stage_tag);
    };
    // acc = alpha * acc when some row moved its reference, then O^T += V^T P^T
    // from V stage S
    auto pv_st = [&](const u32x4 (&pfv)[QB][KB][2], const float (&al)[QB], const PreOps& pre,
                     auto stage_tag) {
      bool moved = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) moved |= al[qb] != 1.f;
      if (__any(moved)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[qb][db] *= al[qb];
      }
      if constexpr (ASMPH > 0) {
        constexpr int S = decltype(stage_tag)::value;
        const uint32_t a0 = lds0 + va[0][0], b0 = lds0 + va[0][1], a1 = lds0 + va[1][0], b1 = lds0 + va[1][1];
        const uint32_t a2 = lds0 + va[2][0], b2 = lds0 + va[2][1], a3 = lds0 + va[3][0], b3 = lds0 + va[3][1];
#define FA2_PV_OPERANDS                                                                                         \
  : [a0] "+v"(acc[0][0]), [a1] "+v"(acc[0][1]), [a2] "+v"(acc[0][2]), [a3] "+v"(acc[0][3])                   \
  : [va0] "v"(a0), [vb0] "v"(b0), [va1] "v"(a1), [vb1] "v"(b1), [va2] "v"(a2), [vb2] "v"(b2), [va3] "v"(a3), \
    [vb3] "v"(b3), [p00] "v"(pfv[0][0][0]), [p01] "v"(pfv[0][0][1]), [p10] "v"(pfv[0][1][0]),                \
    [p11] "v"(pfv[0][1][1]), [o00] "n"(S * TSZ), [o01] "n"(S * TSZ + 16 * KROW),                              \
    [o10] "n"(S * TSZ + 32 * KROW), [o11] "n"(S * TSZ + 48 * KROW)
        if constexpr (BF16) {
          static_assert(ASMPH == 4 || ASMPH == 8, "generated lookaheads: 4, 8");
          if constexpr (ASMPH == 4) asm volatile(FA2_ASM_PV_BF16_L4 FA2_PV_OPERANDS : "memory", FA2_ASM_CLOBBERS_L4);
          else asm volatile(FA2_ASM_PV_BF16_L8 FA2_PV_OPERANDS : "memory", FA2_ASM_CLOBBERS_L8);
        } else {
          static_assert(ASMPH == 4 || ASMPH == 8, "generated lookaheads: 4, 8");
          if constexpr (ASMPH == 4) asm volatile(FA2_ASM_PV_F16_L4 FA2_PV_OPERANDS : "memory", FA2_ASM_CLOBBERS_L4);
          else asm volatile(FA2_ASM_PV_F16_L8 FA2_PV_OPERANDS : "memory", FA2_ASM_CLOBBERS_L8);
        }
#undef FA2_PV_OPERANDS
        return;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int i = (db * KB + kb) * 2 + st;
            u32x4 vf;
            if (i < NPRE) vf = pre[i < NPRE ? i : 0];
            else vf = vread(db, kb, st, stage_tag);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb][db] = E::mfma(vf, pfv[qb][kb][st], acc[qb][db]);
          }
        }
      }
      if constexpr (TL::LOOK > 0) {
        // two transpose reads per MFMA, 2*LOOK reads ahead
        constexpr int NM = NPV - NPRE;
        constexpr int LA = TL::LOOK < NM ? TL::LOOK : NM;
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * LA, 0);
#pragma unroll
        for (int i = 0; i < NM - LA; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, LA + NPRE, 0);
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // one tile: scores, (prefetched P.V operands), softmax, P.V
    auto tile = [&](int j, auto stage_tag) {
      const int key0 = j * BC;
      if (tile_skip(key0)) return;
      f32x16 sv[QB][KB];
      u32x4 pfv[QB][KB][2];
      float al[QB];
      PreOps pre;
      scores_st(sv, stage_tag);
      if constexpr (TL::LOOK > 0) order_scores(std::integral_constant<int, TL::LOOK>{}, I0{});
      if constexpr (NPRE > 0) vpre(pre, stage_tag);
      softmax(sv, key0, tile_masked(key0), pfv, al);
      pv_st(pfv, al, pre, stage_tag);
    };

    if constexpr (TL::PIPE == 11) {
      // ---- half-shifted wave groups over the 3-stage ring -------------------
      // Waves 0-3 (group A) run one phase ahead of waves 4-7 (group B), which
      // share their SIMDs (wave w runs on SIMD w % 4).  In step j group B runs
      // the plain order: scores of tile j, softmax, P.V; group A runs the
      // softmax of tile j (scores computed in step j-1), P.V of tile j, then
      // the scores of tile j+1.  With one barrier per step, one wave's softmax
      // then meets the other wave's MFMAs at the start of the step, and both
      // waves issue MFMAs in its second part.  Group A reads tile j+1 in step
      // j, so every wave waits for its copies of tile j+1 before the barrier
      // of step j (one step of copy lead time); after that barrier the stage
      // of tile j-1 (last read in step j-1) receives tile j+2.
      static_assert(NS == 3 && NW == 8, "half-shifted groups use the 8-wave 3-stage ring");
      const bool ahead = wave < 4;
      f32x16 sa[QB][KB];                          // group A: scores of the next tile
      auto step = [&](int j, auto stage_tag) {
        constexpr int S = decltype(stage_tag)::value;   // == j % 3
        if (j >= 1) {
          FA2_WAIT_VMCNT(0);
          __syncthreads();
        }
        if (j + 2 < nt) dma(j + 2, std::integral_constant<int, (S + 2) % 3>{});
        const int key0 = j * BC;
        if (ahead) {
          if (!tile_skip(key0)) {
            u32x4 pfv[QB][KB][2];
            float al[QB];
            PreOps pre;
            softmax(sa, key0, tile_masked(key0), pfv, al);
            pv_st(pfv, al, pre, stage_tag);
          }
          if (j + 1 < nt && !tile_skip(key0 + BC)) {
            scores_st(sa, std::integral_constant<int, (S + 1) % 3>{});
            if constexpr (TL::LOOK > 0) order_scores(std::integral_constant<int, TL::LOOK>{}, I0{});
          }
        } else {
          tile(j, stage_tag);
        }
      };
      dma(0, I0{});
      if (nt > 1) dma(1, I1{});
      FA2_WAIT_VMCNT(0);
      q_ready();
      __syncthreads();
      if (ahead && !tile_skip(0)) {
        scores_st(sa, I0{});
        if constexpr (TL::LOOK > 0) order_scores(std::integral_constant<int, TL::LOOK>{}, I0{});
      }
      int j = 0;
      for (; j + 3 <= nt; j += 3) {
        step(j, I0{});
        step(j + 1, I1{});
        step(j + 2, I2{});
      }
      if (j < nt) step(j, I0{});
      if (j + 1 < nt) step(j + 1, I1{});
    } else if constexpr (TL::PIPE == 10) {
      // ---- 32-key blocks; softmax threaded between the wave's own MFMAs --------
      // A single wave cannot keep the MFMA pipe full (measured: ≈36 cycles per
      // back-to-back MFMA, ≈42 with operand reads and waits between them, 32
      // when two waves interleave), so both waves of a SIMD must issue MFMAs
      // all the time, and each wave's softmax has to run between its own
      // MFMAs.  Block i = 2t + h is half h of key tile t (ring stage t % 4).
      // Iteration i issues, as one region in a fixed order: the score MFMAs
      // of block i+1 and the P.V MFMAs of block i-1 (16 MFMAs, their LDS
      // operands read RA MFMAs ahead), with the softmax of block i cut into 16
      // chunks placed after them; scheduling barriers keep that order.  The
      // rescale of acc (rare) and the masking of a diagonal or tail block run
      // before the region.  Barrier and copies as in the block pipeline: the
      // barrier before the first read of tile t+1 (iteration 2t+1) publishes
      // tile t+1 and frees the stage of tile t-1 (its V was last read in
      // iteration 2t), which receives tile t+3.
      static_assert(QB == 1 && KB == 2, "the block pipeline assumes 32 rows per wave and 64-key tiles");
      constexpr int RA = TL::PRE > 0 ? TL::PRE : 4;      // MFMA operands read ahead
      static_assert(RA >= 1, "read-ahead");
      int n_eff = N;
      if constexpr (CAUSAL) n_eff = min(N, q_wg + BR);
      const int nb = (n_eff + 31) / 32;          // 32-key blocks this workgroup visits
      auto live = [&](int i) { return i >= 0 && i < nb && !(CAUSAL && 32 * i > q_w + 31); };
      auto masked = [&](int i) { return (32 * i + 32 > N) || (CAUSAL && 32 * i + 31 > q_w); };
      auto koff_of = [&](int blk) { return ((blk >> 1) & 3) * TSZ + (blk & 1) * 32 * KROW; };
      auto kread = [&](int dk, int koff) { return *(const u32x4*)(smem + (ka[dk] + koff)); };
      auto vtread = [&](int db, int st, int voff) {
        const u32x2 lo = lds_read_tr16(smem + (va[db][0] + voff) + 16 * st * KROW);
        const u32x2 hi = lds_read_tr16(smem + (va[db][1] + voff) + 16 * st * KROW);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      auto rescale = [&](float al) {
        if (__any(al != 1.f)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[0][db] *= al;
        }
      };
      auto mask_blk = [&](f32x16& sv, int i) {
        const int q = q_w + lr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
          const bool vis = key < N && (!CAUSAL || key <= q);
          sv[r] = vis ? sv[r] * c : -INFINITY;
        }
      };
      f32x16 sbuf[2];
      u32x4 pbuf[2][2];
      float abuf[2];
      // plain (unthreaded) pieces for the first and last blocks
      auto sblk = [&](f32x16& sv, int koff) {
        sv = f32x16{};
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) sv = E::mfma(kread(dk, koff), qf[0][dk], sv);
      };
      auto pvblk = [&](const u32x4 (&p)[2], int voff) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int st = 0; st < 2; ++st) acc[0][db] = E::mfma(vtread(db, st, voff), p[st], acc[0][db]);
      };
      auto soft_plain = [&](const f32x16& sv, float cc, u32x4 (&p)[2], float& al) {
        float e0 = fmaxf(sv[0], sv[1]), e1 = fmaxf(sv[2], sv[3]);
#pragma unroll
        for (int r = 4; r < 16; r += 4) {
          e0 = fmaxf(e0, fmaxf(sv[r], sv[r + 1]));
          e1 = fmaxf(e1, fmaxf(sv[r + 2], sv[r + 3]));
        }
        const float m_tile = max_halves(fmaxf(e0, e1)) * cc;
        const float m_old = m_run[0];
        const float m_new = (m_tile > m_old + kLazyRescale) ? m_tile : m_old;
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        al = __builtin_amdgcn_exp2f(m_old - m_use);
        m_run[0] = m_new;
        float rs0 = 0.f, rs1 = 0.f, pe[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          pe[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[u], cc, -m_use));
          if (u & 1) rs1 += pe[u]; else rs0 += pe[u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) p[u >> 2][u & 3] = E::pack(pe[2 * u], pe[2 * u + 1]);
        l_run[0] = l_run[0] * al + (rs0 + rs1);
      };
      // iteration i = 2t + H, i >= 1
      auto iter = [&](int t, auto half_tag) {
        constexpr int H = decltype(half_tag)::value;
        constexpr int C = H, O = 1 - H;         // buffers of block i and of blocks i +- 1
        const int i = 2 * t + H;
        if constexpr (H == 1) {
          if (t + 1 < nt) {
            if (t + 2 < nt) FA2_WAIT_VMCNT(2 * NIW); else FA2_WAIT_VMCNT(0);
            __syncthreads();
            if (t + 3 < nt) {
              switch ((t + 3) & 3) {
                case 0: dma(t + 3, I0{}); break;
                case 1: dma(t + 3, I1{}); break;
                case 2: dma(t + 3, I2{}); break;
                default: dma(t + 3, I3{}); break;
              }
            }
          }
        }
        const bool prev = live(i - 1), cur = live(i);
        if (!prev) return;                        // past this wave's diagonal
        rescale(abuf[O]);
        const int voff = koff_of(i - 1);
        if (!cur) {                               // this wave's last P.V
          pvblk(pbuf[O], voff);
          return;
        }
        const bool msk = masked(i);
        if (msk) mask_blk(sbuf[C], i);
        const float cc = msk ? 1.f : c;
        const int koff = koff_of(i + 1);          // past the end: stale LDS, never used
        // ---- the threaded region ----
        f32x16& sv = sbuf[C];
        f32x16& sn = sbuf[O];
        constexpr int NM = DK + 2 * DB;           // MFMAs of the region: DK score, 2*DB P.V
        u32x4 opnd[NM];                           // their operands: K fragments, then V^T fragments
        auto read_op = [&](auto m_tag) {
          constexpr int M = decltype(m_tag)::value;
          if constexpr (M < DK) opnd[M] = kread(M, koff);
          else opnd[M] = vtread((M - DK) >> 1, (M - DK) & 1, voff);
        };
        auto mfma_op = [&](auto m_tag) {
          constexpr int M = decltype(m_tag)::value;
          if constexpr (M < DK) {
            sn = M == 0 ? E::mfma(opnd[M], qf[0][M], f32x16{}) : E::mfma(opnd[M], qf[0][M], sn);
          } else {
            constexpr int db = (M - DK) >> 1, st = (M - DK) & 1;
            acc[0][db] = E::mfma(opnd[M], pbuf[O][st], acc[0][db]);
          }
        };
        float e0, e1, m_use, rs0 = 0.f, rs1 = 0.f, pe[16];
        auto soft_chunk = [&](auto m_tag) {
          constexpr int M = decltype(m_tag)::value;
          if constexpr (M == 0) {
            e0 = fmaxf(sv[0], sv[1]);
            e1 = fmaxf(sv[2], sv[3]);
            e0 = fmaxf(e0, fmaxf(sv[4], sv[5]));
            e1 = fmaxf(e1, fmaxf(sv[6], sv[7]));
          } else if constexpr (M == 1) {
            e0 = fmaxf(e0, fmaxf(sv[8], sv[9]));
            e1 = fmaxf(e1, fmaxf(sv[10], sv[11]));
            e0 = fmaxf(e0, fmaxf(sv[12], sv[13]));
            e1 = fmaxf(e1, fmaxf(sv[14], sv[15]));
          } else if constexpr (M == 2) {
            const float m_tile = max_halves(fmaxf(e0, e1)) * cc;
            const float m_old = m_run[0];
            const float m_new = (m_tile > m_old + kLazyRescale) ? m_tile : m_old;
            m_use = (m_new == -INFINITY) ? 0.f : m_new;
            abuf[C] = __builtin_amdgcn_exp2f(m_old - m_use);
            m_run[0] = m_new;
          } else if constexpr (M >= 3 && M < 11) {
            constexpr int u = 2 * (M - 3);
            pe[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[u], cc, -m_use));
            pe[u + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[u + 1], cc, -m_use));
            rs0 += pe[u];
            rs1 += pe[u + 1];
          } else if constexpr (M >= 11 && M < 15) {
            constexpr int u = 2 * (M - 11);
            pbuf[C][u >> 2][u & 3] = E::pack(pe[2 * u], pe[2 * u + 1]);
            pbuf[C][(u + 1) >> 2][(u + 1) & 3] = E::pack(pe[2 * u + 2], pe[2 * u + 3]);
          } else if constexpr (M == 15) {
            l_run[0] = l_run[0] * abuf[C] + (rs0 + rs1);
          }
        };
        // slot m: MFMA m, softmax chunks [16m/NM, 16(m+1)/NM), operand read m+RA
        static_assert(RA < NM, "read-ahead");
        static_for<0, RA>([&](auto m) { read_op(m); });
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, NM>([&](auto m) {
          constexpr int M = decltype(m)::value;
          mfma_op(m);
          static_for<16 * M / NM, 16 * (M + 1) / NM>([&](auto c) { soft_chunk(c); });
          if constexpr (M + RA < NM) read_op(std::integral_constant<int, M + RA>{});
          __builtin_amdgcn_sched_barrier(0);
        });
      };
      const int np = min(nt, 3);                  // tiles copied before the loop
      dma(0, I0{});
      if (np > 1) dma(1, I1{});
      if (np > 2) dma(2, I2{});
      if (np == 3) FA2_WAIT_VMCNT(4 * NIW); else if (np == 2) FA2_WAIT_VMCNT(2 * NIW); else FA2_WAIT_VMCNT(0);
      q_ready();
      __syncthreads();
      // iteration 0: scores of blocks 0 and 1, softmax of block 0 (every wave
      // sees key 0)
      sblk(sbuf[0], 0);
      sblk(sbuf[1], 32 * KROW);
      {
        const bool msk = masked(0);
        if (msk) mask_blk(sbuf[0], 0);
        soft_plain(sbuf[0], msk ? 1.f : c, pbuf[0], abuf[0]);
      }
      iter(0, I1{});
      for (int t = 1; t < nt; ++t) {
        iter(t, I0{});
        iter(t, I1{});
      }
      // the P.V of the last block (iteration 2*nt)
      iter(nt, I0{});
    } else if constexpr (TL::PIPE == 9) {
      // ---- ping-pong over the direct-copy ring --------------------------------
      // The NW waves form two groups of NW/2; wave w runs on SIMD w % 4, so
      // each SIMD holds one wave of each group.  Time is cut into half-steps
      // separated by barriers.  In half-step h a group whose phase h - g is
      // even runs its MFMA phase for tile t = (h - g) / 2 (P.V of tile t-1,
      // then the scores of tile t); a group whose phase is odd runs the softmax
      // of tile (h - g - 1) / 2.  The groups are always in opposite phases, so
      // on every SIMD one wave feeds the MFMA pipe while the other keeps the
      // VALU busy.  Tile u sits in stage u % 4: its K is read in half-steps 2u
      // and 2u+1, its V in 2u+2 and 2u+3.  At the barrier opening half-step
      // 2k every wave's copies of tile k have landed, and tile k-2 (last read
      // in half-step 2k-1) is dead: its stage receives tile k+2.
      static_assert(NW == 8, "ping-pong pairs the two waves of every SIMD");
      const int grp = wave >> 2;
      f32x16 sc[QB][KB];
      u32x4 pf[QB][KB][2];
      float al[QB];
      PreOps pre;
      const int nh = 2 * nt + 2;                    // half-steps
      auto half = [&](int h, auto r_tag) {
        constexpr int R = decltype(r_tag)::value;   // h % 8
        if (h >= nh) return;
        if constexpr (R % 2 == 0) {
          const int k = h >> 1;
          if (k >= 1 && k < nt) {
            if (k + 1 < nt) FA2_WAIT_VMCNT(2 * NIW); else FA2_WAIT_VMCNT(0);
          }
        }
        __syncthreads();
        if constexpr (R % 2 == 0) {
          const int k = h >> 1;
          if (k >= 1 && k + 2 < nt) dma(k + 2, std::integral_constant<int, (R / 2 + 2) % 4>{});
        }
        if (grp == (R & 1)) {
          // MFMA phase for tile t (stage ST)
          constexpr int ST = (R / 2) % 4;
          const int t = (h - grp) >> 1;
          if (t >= 1 && !tile_skip((t - 1) * BC)) pv_st(pf, al, pre, std::integral_constant<int, (ST + 3) % 4>{});
          if (t < nt && !tile_skip(t * BC)) {
            scores_st(sc, std::integral_constant<int, ST>{});
            if constexpr (TL::LOOK > 0) order_scores(std::integral_constant<int, TL::LOOK>{}, I0{});
          }
        } else {
          // softmax phase for tile t (stage SST); the wave's LDS port is idle
          // here, so the first PRE V^T operands of its next P.V (tile t) are
          // read now
          constexpr int SST = (R & 1) ? ((R - 1) / 2) % 4 : (R / 2 + 3) % 4;
          const int t = (h - grp - 1) >> 1;
          if (h - grp >= 1 && t < nt && !tile_skip(t * BC)) {
            if constexpr (NPRE > 0) vpre(pre, std::integral_constant<int, SST>{});
            softmax(sc, t * BC, tile_masked(t * BC), pf, al);
          }
        }
      };
      dma(0, I0{});
      if (nt > 1) dma(1, I1{});
      if (nt > 2) dma(2, I2{});
      // Q and tile 0 have landed when only the copies of tiles 1, 2 remain
      if (nt > 2) FA2_WAIT_VMCNT(4 * NIW); else if (nt > 1) FA2_WAIT_VMCNT(2 * NIW); else FA2_WAIT_VMCNT(0);
      q_ready();
      for (int h = 0; h < nh; h += 8) {
        half(h, I0{});
        half(h + 1, I1{});
        half(h + 2, I2{});
        half(h + 3, I3{});
        half(h + 4, std::integral_constant<int, 4>{});
        half(h + 5, std::integral_constant<int, 5>{});
        half(h + 6, std::integral_constant<int, 6>{});
        half(h + 7, std::integral_constant<int, 7>{});
      }
    } else if constexpr (TL::PIPE != 7) {
      auto step = [&](int j, auto stage_tag) {
        constexpr int S = decltype(stage_tag)::value;   // == j % NS
        // this wave's copies of tile j are done once at most the copies of the
        // tiles issued after it (NS-2 of them, 2*NIW instructions each) remain
        if constexpr (NS == 3) {
          if (j + 1 < nt) FA2_WAIT_VMCNT(2 * NIW); else FA2_WAIT_VMCNT(0);
        } else {
          FA2_WAIT_VMCNT(0);
        }
        // every wave's tile j has landed and every wave has finished tile j-1,
        // so stage (j-1)%NS == (j+NS-1)%NS may be refilled
        __syncthreads();
        if (j + NS - 1 < nt) dma(j + NS - 1, std::integral_constant<int, (S + NS - 1) % NS>{});
        tile(j, stage_tag);
      };
      dma(0, I0{});
      if (NS == 3 && nt > 1) dma(1, std::integral_constant<int, 1 % NS>{});
      // Q fragments were loaded before the copies: wait for them only
      if (NS == 3 && nt > 1) FA2_WAIT_VMCNT(4 * NIW); else FA2_WAIT_VMCNT(2 * NIW);
      q_ready();
      int j = 0;
      for (; j + NS <= nt; j += NS) {
        step(j, I0{});
        step(j + 1, I1{});
        if constexpr (NS == 3) step(j + 2, std::integral_constant<int, 2 % NS>{});
      }
      if (j < nt) step(j, I0{});
      if (NS == 3 && j + 1 < nt) step(j + 1, I1{});
    } else {
      // 4-stage ring, one barrier per pair of tiles.  At the barrier before
      // tiles j, j+1 (j even) every wave's copies of both have landed and
      // every wave has finished tiles j-2, j-1, whose stages then receive
      // tiles j+2, j+3.  Within a pair the waves drift freely.
      static_assert(NS == 4, "pair-barrier loop uses 4 stages");
      static_assert(4 * NIW < 64, "vmcnt range");
      auto pair = [&](int j, auto stage_tag) {
        constexpr int S = decltype(stage_tag)::value;   // == j % 4, even
        // tiles j, j+1 must have landed; j+2, j+3 are not issued yet
        FA2_WAIT_VMCNT(0);
        __syncthreads();
        if (j + 2 < nt) dma(j + 2, std::integral_constant<int, (S + 2) % 4>{});
        if (j + 3 < nt) dma(j + 3, std::integral_constant<int, (S + 3) % 4>{});
        tile(j, stage_tag);
        if (j + 1 < nt) tile(j + 1, std::integral_constant<int, S + 1>{});
      };
      dma(0, I0{});
      if (nt > 1) dma(1, I1{});
      FA2_WAIT_VMCNT(0);
      q_ready();
      int j = 0;
      for (; j + 4 <= nt; j += 4) {
        pair(j, I0{});
        pair(j + 2, I2{});
      }
      if (j < nt) pair(j, I0{});
      if (j + 2 < nt) pair(j + 2, I2{});
    }
  } else if constexpr (TL::PIPE == 3) {
    // ---- ping-pong schedule -------------------------------------------------
    // The NW waves form two groups of NW/2; wave i runs on SIMD i % 4, so with
    // NW = 8 each SIMD holds one wave of each group.  Time is cut into
    // half-steps separated by barriers.  In half-step h a group whose phase
    // h - g is even runs its MFMA phase for tile t = (h - g) / 2 (P.V of tile
    // t-1, then the scores of tile t); a group whose phase is odd runs its
    // softmax phase for tile (h - g - 1) / 2.  The two groups are always in
    // opposite phases, so on every SIMD one wave feeds the MFMA pipe while the
    // other keeps the VALU busy.
    //   K_t lives in K stage t&1, V_t in V stage t&1.  Group 1 writes K_{t+2}
    //   in its softmax phase of tile t (half-step 2t+2; K_t was last read in
    //   half-step 2t+1) and then fetches K_{t+3}; group 0 writes V_t in its
    //   softmax phase of tile t (half-step 2t+1; V_{t-2} was last read in
    //   half-step 2t-1) and fetches V_{t+1}.  Every global load thus has two
    //   half-steps to land.
    static_assert(NW % 2 == 0, "ping-pong needs an even number of waves");
    constexpr int TG = T / 2;          // threads per group
    constexpr int CHG = CH / TG;       // 16-byte chunks per thread and tile
    static_assert(CH % TG == 0, "tile copy must split evenly over a group");
    const int grp = wave / (NW / 2);
    const int gtid = tid - grp * TG;
    u32x4 gst[CHG];
    const __amdgpu_buffer_rsrc_t grs = grp ? kr : vr;
    auto gload = [&](int key0) {
#pragma unroll
      for (int it = 0; it < CHG; ++it) {
        const int e = gtid + it * TG;
        const int row = e / (D / 8), ch = e % (D / 8);
        gst[it] = __builtin_amdgcn_raw_buffer_load_b128(grs, (uint32_t)((key0 + row) * KROW + ch * 16), 0, 0);
      }
    };
    auto gstore = [&](int stage) {
      uint8_t* base = grp ? kring + stage * KSTAGE : vring + stage * VSTAGE;
      const int pitch = grp ? KP : VP;
#pragma unroll
      for (int it = 0; it < CHG; ++it) {
        const int e = gtid + it * TG;
        const int row = e / (D / 8), ch = e % (D / 8);
        *(u32x4*)(base + row * pitch + ch * 16) = gst[it];
      }
    };
    // prologue: K_0, K_1 into LDS; group 0 holds V_0, group 1 holds K_2
    load_k(0);
    store_k(0);
    if (nt > 1) {
      load_k(BC);
      store_k(1);
    }
    if (grp == 0) gload(0);
    else if (nt > 2) gload(2 * BC);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    f32x16 sc[QB][KB];
    u32x4 pf[QB][KB][2];
    float alpha[QB];
    for (int h = 0; h < 2 * nt + 2; ++h) {
      const int ph = h - grp;
      if (ph >= 0 && (ph & 1) == 0) {
        const int t = ph >> 1;
        __builtin_amdgcn_s_setprio(1);
        if (t >= 1 && !tile_skip((t - 1) * BC)) rescale_pv(vring + ((t - 1) & 1) * VSTAGE, pf, alpha);
        if (t < nt && !tile_skip(t * BC)) scores(kring + (t & 1) * KSTAGE, sc);
        __builtin_amdgcn_s_setprio(0);
      } else if (ph >= 1) {
        const int t = (ph - 1) >> 1;
        if (t < nt) {
          if (!tile_skip(t * BC)) softmax(sc, t * BC, tile_masked(t * BC), pf, alpha);
          if (grp == 0) {
            gstore(t & 1);                         // V_t
            if (t + 1 < nt) gload((t + 1) * BC);   // V_{t+1}
          } else {
            if (t + 2 < nt) gstore(t & 1);         // K_{t+2}
            if (t + 3 < nt) gload((t + 3) * BC);   // K_{t+3}
          }
        }
      }
      __syncthreads();
    }
  } else {
    // ---- software-pipelined loop ------------------------------------------
    // Iteration j: scores of tile j+1 (K_{j+1} from K stage (j+1)&1) are
    // issued together with the softmax of tile j, then acc += V_j P_j (V
    // stage j&1).  K_{j+2} and V_{j+1} are fetched during the iteration and
    // written to K stage j&1 and V stage (j+1)&1, which nobody reads in
    // iteration j; one barrier per iteration publishes them.
    const int nclean = CAUSAL ? min(q_wg, N) / BC : N / BC;  // tiles no wave masks
    const int nfast = min(nclean, nt - 1);
    load_k(0);
    load_v(0);
    store_k(0);
    store_v(0);
    if (nt > 1) {
      load_k(BC);
      store_k(1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    f32x16 sc[QB][KB];
    if (!tile_skip(0)) scores(kring, sc);

    auto iteration = [&](int j, auto has_next_tag, auto fast_tag) {
      constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
      constexpr bool FAST = decltype(fast_tag)::value;
      const int key0 = j * BC;
      const bool load2 = HAS_NEXT && j + 2 < nt;
      if (load2) load_k(key0 + 2 * BC);
      if (HAS_NEXT) load_v(key0 + BC);
      f32x16 sn[QB][KB];
      u32x4 pf[QB][KB][2];
      float alpha[QB];
      if constexpr (FAST) {
        // no mask, no skip: one basic block for the MFMAs and the softmax
        scores(kring + ((j + 1) & 1) * KSTAGE, sn);
        softmax(sc, key0, false, pf, alpha);
        if constexpr (TL::PIPE == 2) {
          // issue order: the tile loads, then (LDS read, MFMA, VALU x n) per
          // score MFMA, so the softmax VALU work fills the MFMA shadow
#pragma unroll
          for (int i = 0; i < 2 * CH_T; ++i) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
#pragma unroll
          for (int i = 0; i < QB * KB * DK; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuPerMfma, 0);
          }
        }
        rescale_pv(vring + (j & 1) * VSTAGE, pf, alpha);
      } else {
        if (HAS_NEXT && !tile_skip(key0 + BC)) scores(kring + ((j + 1) & 1) * KSTAGE, sn);
        if (!tile_skip(key0)) {
          softmax(sc, key0, tile_masked(key0), pf, alpha);
          rescale_pv(vring + (j & 1) * VSTAGE, pf, alpha);
        }
      }
      if (load2) store_k(j & 1);
      if (HAS_NEXT) store_v((j + 1) & 1);
      __syncthreads();
      if constexpr (HAS_NEXT) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) sc[qb][kb] = sn[qb][kb];
      }
    };
    int j = 0;
    for (; j < nfast; ++j) iteration(j, std::true_type{}, std::true_type{});
    for (; j < nt - 1; ++j) iteration(j, std::true_type{}, std::false_type{});
    iteration(nt - 1, std::false_type{}, std::false_type{});
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ---------------------
  const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((uint16_t*)a.o + head_off), 0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t lr_ = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.lse + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q_w + qb * 32 + lr;
    const float l = sum_halves(l_run[qb]);
    const float inv = 1.f / l;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = E::pack(acc[qb][db][4 * i + 0] * inv, acc[qb][db][4 * i + 1] * inv);
        w[1] = E::pack(acc[qb][db][4 * i + 2] * inv, acc[qb][db][4 * i + 3] * inv);
        const int d = 32 * db + 8 * i + 4 * lh;
        __builtin_amdgcn_raw_buffer_store_b64(w, orr, (uint32_t)(row * KROW + d * 2), 0, 0);
      }
    }
    if (lh == 0) {
      const float lse = (m_run[qb] + log2f(l)) * 0.69314718055994530942f;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), lr_, (uint32_t)(row * 4), 0, 0);
    }
  }
}

}  // namespace fa2
