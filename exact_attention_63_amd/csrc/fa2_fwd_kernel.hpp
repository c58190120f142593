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
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;

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

// LDS read of 16 bytes at a byte address of the workgroup's allocation.
__device__ __forceinline__ u32x4 lds_load_b128(uint32_t addr) {
  return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)addr;
}

// Bytes of LDS a wave needs to stage its output rows (store_o128_staged).
constexpr int kStageBytes = 4096;

// The O^T accumulators of a wave's 32 rows (d = 128; lane (row lr, half lh)
// holds d = 32 db + 8 (r / 4) + 4 lh + r % 4 in register r of block db) times
// scale, rounded to 16 bits (bf16 or fp16), stored to rows q_w .. q_w + 31 of
// the buffer orr (row stride 256 bytes; rows past its end are dropped).  The
// rows go through the wave's 4 KiB of LDS at stage (4 KiB aligned, nobody
// else's while this runs), 16 at a time, so that each store writes whole
// rows: lane L stores bytes [16 (L % 16), +16) of row L / 16 of a group of 4.
// Stored straight from the accumulator layout, every row would arrive in 16
// pieces of 16 bytes from 16 instructions; with all workgroups storing at once
// those partial-line writes held the stores for thousands of cycles.
template <bool BF16>
__device__ __forceinline__ void store_o128_staged(__amdgpu_buffer_rsrc_t orr, int q_w, int lane, const f32x16& acc0,
                                                  const f32x16& acc1, const f32x16& acc2, const f32x16& acc3,
                                                  float scale, uint8_t* stage) {
  using E = Elem<BF16>;
  const int lr = lane & 31, lh = lane >> 5;
  // Row r (of 16) at stage + 256 r, its 16-byte chunk c at 16 (c ^ r): the 16
  // rows a half-wave writes, and the 4 rows a read covers, hit distinct banks.
  // Chunk k = 4 db + i of row lr is d = 8 k .. 8 k + 7, its half lh from this
  // lane (accumulator registers 4 i .. 4 i + 3 of block db).  The row, chunk
  // and half occupy disjoint address bits, so every address is one per-lane
  // base XOR an immediate; the empty asm keeps the compiler from hoisting
  // per-lane addresses out of a caller's loop.
  const uint32_t sbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)stage;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((lr >> 4) == half) {
      const uint32_t r = lr & 15;
      uint32_t wb = sbase | (256u * r + 16u * r + 8u * (uint32_t)lh);   // chunk k at wb ^ 16 k
      asm volatile("" : "+v"(wb));
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const f32x16& acc = db == 0 ? acc0 : db == 1 ? acc1 : db == 2 ? acc2 : acc3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 v;
          v[0] = E::pack(acc[4 * i + 0] * scale, acc[4 * i + 1] * scale);
          v[1] = E::pack(acc[4 * i + 2] * scale, acc[4 * i + 3] * scale);
          *(__attribute__((address_space(3))) u32x2*)(uintptr_t)(wb ^ (16u * (4 * db + i))) = v;
        }
      }
    }
    // lane L reads chunk c = L % 16 of row r = 4 g + L / 16, at
    // (rb ^ 64 g) + 1024 g with rb = stage + 256 (L / 16) + 16 (c ^ (L / 16))
    const uint32_t rr = (uint32_t)lane >> 4, c = (uint32_t)lane & 15;
    uint32_t rb = sbase | (256u * rr + 16u * (c ^ rr));
    asm volatile("" : "+v"(rb));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4 x = lds_load_b128((rb ^ (64u * g)) + 1024u * g);
      __builtin_amdgcn_raw_buffer_store_b128(x, orr, (uint32_t)((q_w + 16 * half + 4 * g + (int)rr) * 256 + 16 * (int)c),
                                             0, 0);
    }
  }
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
// The same copy as inline assembly: the compiler then does not track it at
// all, and the kernel's own ordering is the only one: each wave waits for its
// copies of a stage with s_waitcnt vmcnt, then a barrier publishes the stage.  M0 holds the LDS destination; one wait state
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

// ds_read_b64_tr_b16: transpose read of 16-bit elements (see the V fragment
// comment in the kernel for the lane mapping).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Causal grids: workgroup i -> (head bh, query block qblk).  Workgroups are
// dealt to the 8 XCDs round robin (workgroup i runs on XCD i % 8), so with
// B*H a multiple of 8 the heads h with h % 8 == x all run on XCD x.  XCD x
// takes them in groups of G heads, G = 32 / (query blocks per head) (at
// least 1): about one block per CU of the XCD (32).  Within a group the
// blocks go level by level, heaviest first.  The first group's blocks start
// together, and as they finish (lightest first) the next group's blocks
// start heaviest first, so every CU's total comes out about the same; the
// workgroups an XCD runs at a time belong to one or two groups and share
// their K and V in its L2 (N = 16384: 2.9x fewer L2 misses than all heads
// of an XCD level by level).  Otherwise all heads go level by level.
__device__ __forceinline__ void causal_item(int i, int BH, int nqb, int& bh, int& qblk) {
  const int G = nqb >= 32 ? 1 : 32 / nqb;
  if (BH % 8 == 0 && (BH / 8) % G == 0) {
    const int s = i / 8;                 // the s-th workgroup of XCD i % 8
    const int per = G * nqb;             // blocks of one group
    const int g = s / per, r = s % per;
    bh = (g * G + r % G) * 8 + i % 8;
    qblk = nqb - 1 - r / G;
  } else {
    bh = i % BH;
    qblk = nqb - 1 - i / BH;
  }
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
//   RING: 0 = K/V tiles staged through registers into a 2-stage padded LDS
//         ring; 2 or 3 = K/V copied straight from HBM into a ring of that
//         many LDS stages (buffer_load ... lds), swizzled unpadded rows
//   LOOK (direct-copy rings): keep this many score-MFMA operand reads in
//         flight ahead of the MFMAs (0: leave the order to the compiler)
//   SWEXP: the softmax's 2^x from sw_exp2 (FMA pipe) for every score (1), for
//         every other score (2), or from v_exp_f32 only (0)
template <int NW_, int QB_, int KB_, int WPE_, int RING_ = 0, int LOOK_ = 0, int SWEXP_ = 0>
struct Tile {
  static constexpr int NW = NW_, QB = QB_, KB = KB_, WPE = WPE_;
  static constexpr int RING = RING_, LOOK = LOOK_, SWEXP = SWEXP_;
  static_assert(RING == 0 || RING == 2 || RING == 3, "ring stages");
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
  // direct-copy rings: NS stages of unpadded, XOR-swizzled [key][d] K and V tiles
  constexpr int TSZ = BC * KROW;        // bytes of one unpadded K (or V) tile
  constexpr int NS = TL::RING;
  constexpr int SMEM = NS > 0 ? NS * 2 * TSZ : 2 * STAGE;
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
  // Causal: causal_item (heaviest query blocks first, a head's blocks on one
  // XCD).
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

  if constexpr (TL::RING == 0) {
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
  } else {
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
        lds_dma16(kr, smem + S * TSZ + dst, dsrc[k], base);
        lds_dma16(vr, smem + (NS + S) * TSZ + dst, dsrc[k], base);
      }
    };
    // The compiler does not relate the copies to Q, so it may believe the Q
    // loads are still in flight inside the loop and wait for them (and so for
    // every copy issued after them) there.  Once the explicit wait has covered
    // Q, pass the Q registers through an empty statement: the compiler's own
    // wait for them lands here, before the loop.
    auto q_ready = [&]() {
      static_assert(QB * DK == 4 || QB * DK == 8, "Q fragment count");
      const u32x4* qq = &qf[0][0];
      if constexpr (QB * DK == 4) {
        asm volatile("" ::"v"(qq[0]), "v"(qq[1]), "v"(qq[2]), "v"(qq[3]));
      } else {
        asm volatile("" ::"v"(qq[0]), "v"(qq[1]), "v"(qq[2]), "v"(qq[3]), "v"(qq[4]), "v"(qq[5]), "v"(qq[6]),
                     "v"(qq[7]));
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
    auto scores_st = [&](f32x16 (&sv)[QB][KB], auto stage_tag) {
      constexpr int S = decltype(stage_tag)::value;
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
    // MFMA per further read
    auto order_scores = [&]() {
      constexpr int LOOK = TL::LOOK, NM = QB * KB * DK, NR = KB * DK;
      static_assert(QB == 1, "read lookahead assumes one fragment per MFMA");
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LOOK, 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (i < NR - LOOK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
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
    // acc = alpha * acc when some row moved its reference, then O^T += V^T P^T
    // from V stage S
    auto pv_st = [&](const u32x4 (&pfv)[QB][KB][2], const float (&al)[QB], auto stage_tag) {
      bool moved = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) moved |= al[qb] != 1.f;
      if (__any(moved)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[qb][db] *= al[qb];
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const u32x4 vf = vread(db, kb, st, stage_tag);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb][db] = E::mfma(vf, pfv[qb][kb][st], acc[qb][db]);
          }
        }
      }
      if constexpr (TL::LOOK > 0) {
        // two transpose reads per MFMA, 2*LOOK reads ahead
        constexpr int LA = TL::LOOK < NPV ? TL::LOOK : NPV;
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * LA, 0);
#pragma unroll
        for (int i = 0; i < NPV - LA; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, LA, 0);
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // one tile: scores, softmax, P.V
    auto tile = [&](int j, auto stage_tag) {
      const int key0 = j * BC;
      if (tile_skip(key0)) return;
      f32x16 sv[QB][KB];
      u32x4 pfv[QB][KB][2];
      float al[QB];
      scores_st(sv, stage_tag);
      if constexpr (TL::LOOK > 0) order_scores();
      softmax(sv, key0, tile_masked(key0), pfv, al);
      pv_st(pfv, al, stage_tag);
    };
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
