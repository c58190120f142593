// fa2_api.hip -- host side of the C ABI declared in include/fa2.h: argument
// validation, the tile-variant table and the kernel launch.
//
// A forward call enqueues one kernel, a backward call three; each returns
// after enqueueing.  It allocates nothing (the method
// needs O(N) memory: only the inputs and outputs), keeps no state besides
// constant tables, and validates every argument before touching the HIP
// runtime, so an invalid call has no effect.
#include <stdint.h>
#include <algorithm>
#include <atomic>
#include <string.h>

#include "fa2.h"
#include "fa2_fwd_kernel.hpp"
#include "fa2_bwd_kernel.hpp"
#include "fa2_fwd_roles.hpp"
#include "fa2_fwd_sched.hpp"

#define FA2_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using fa2::Args;
using fa2::Tile;

typedef void (*kernel_fn)(Args);

// One tile configuration and its kernels for every (dtype, d, causal).
struct Variant {
  const char* name;
  int threads;
  int rows_per_block;     // BR
  kernel_fn fn[2][2][2];  // [bf16][d == 128][causal]
  // persistent kernel for d = 128, non-causal, N % 256 == 0 (one workgroup
  // per CU); null where the variant has none
  kernel_fn persist[2];   // [bf16]
};

template <class TL>
constexpr Variant make_variant(const char* name) {
  return Variant{name,
                 TL::THREADS,
                 TL::BR,
                 {{{fa2::fa2_fwd_kernel<false, 64, false, TL>, fa2::fa2_fwd_kernel<false, 64, true, TL>},
                   {fa2::fa2_fwd_kernel<false, 128, false, TL>, fa2::fa2_fwd_kernel<false, 128, true, TL>}},
                  {{fa2::fa2_fwd_kernel<true, 64, false, TL>, fa2::fa2_fwd_kernel<true, 64, true, TL>},
                   {fa2::fa2_fwd_kernel<true, 128, false, TL>, fa2::fa2_fwd_kernel<true, 128, true, TL>}}}};
}

// The role-split kernel (fa2_fwd_roles.hpp): 8 waves, 128 queries per workgroup.
constexpr Variant make_roles_variant(const char* name) {
  return Variant{name,
                 512,
                 128,
                 {{{fa2::fa2_fwd_roles_kernel<false, 64, false>, fa2::fa2_fwd_roles_kernel<false, 64, true>},
                   {fa2::fa2_fwd_roles_kernel<false, 128, false>, fa2::fa2_fwd_roles_kernel<false, 128, true>}},
                  {{fa2::fa2_fwd_roles_kernel<true, 64, false>, fa2::fa2_fwd_roles_kernel<true, 64, true>},
                   {fa2::fa2_fwd_roles_kernel<true, 128, false>, fa2::fa2_fwd_roles_kernel<true, 128, true>}}}};
}

// The scheduled kernel (fa2_fwd_sched.hpp) at d = 128; d = 64 runs the
// 128-key-tile kernel of the same workgroup shape (8 waves, 256 rows).
constexpr Variant make_sched_variant(const char* name) {
  using D64 = Tile<8, 1, 4, 2, 5, 4>;
  return Variant{name,
                 512,
                 fa2::kSchedRows,
                 {{{fa2::fa2_fwd_kernel<false, 64, false, D64>, fa2::fa2_fwd_kernel<false, 64, true, D64>},
                   {fa2::fa2_fwd_sched_kernel<false, false>, fa2::fa2_fwd_sched_kernel<false, true>}},
                  {{fa2::fa2_fwd_kernel<true, 64, false, D64>, fa2::fa2_fwd_kernel<true, 64, true, D64>},
                   {fa2::fa2_fwd_sched_kernel<true, false>, fa2::fa2_fwd_sched_kernel<true, true>}}},
                 {nullptr, nullptr}};
}

// ... with its persistent form where the shape allows it
constexpr Variant make_sched_persist_variant(const char* name) {
  Variant v = make_sched_variant(name);
  v.persist[0] = fa2::fa2_fwd_sched_persist_kernel<false>;
  v.persist[1] = fa2::fa2_fwd_sched_persist_kernel<true>;
  return v;
}

// Index 0 is the tuned default; it is resolved per (dtype, d, causal) by
// default_variant() below.
const Variant kVariants[] = {
    {"default", 0, 0, {}},
    make_variant<Tile<4, 1, 2, 2>>("w4_q32_k64_occ2"),   // 4 waves x 32 rows, 64-key tiles, 2 waves/SIMD
    make_variant<Tile<4, 2, 2, 1>>("w4_q64_k64_occ1"),   // 4 waves x 64 rows, 64-key tiles, 1 wave/SIMD
    make_variant<Tile<8, 1, 2, 2>>("w8_q32_k64_occ2"),   // 8 waves x 32 rows, 64-key tiles, 2 waves/SIMD
    make_variant<Tile<4, 1, 2, 2, 1>>("w4_q32_k64_occ2_pipe"),    // variant 1, software-pipelined loop
    make_variant<Tile<8, 1, 2, 2, 1>>("w8_q32_k64_occ2_pipe"),    // variant 3, software-pipelined loop
    make_variant<Tile<4, 1, 2, 2, 2>>("w4_q32_k64_occ2_ilv"),     // variant 4 + MFMA/VALU interleave
    make_variant<Tile<8, 1, 2, 2, 2>>("w8_q32_k64_occ2_ilv"),     // variant 5 + MFMA/VALU interleave
    make_variant<Tile<8, 1, 2, 2, 3>>("w8_q32_k64_pingpong"),     // two 4-wave groups in opposite phases
    make_variant<Tile<8, 1, 2, 2, 4>>("w8_q32_k64_dma3"),         // direct global->LDS copies, 3 stages
    make_variant<Tile<4, 1, 2, 2, 5>>("w4_q32_k64_dma2"),         // 4 waves, 2 stages: two workgroups per CU
    make_variant<Tile<8, 1, 2, 2, 4, 4>>("w8_q32_k64_dma3_look4"), // dma3 + 4 operand reads ahead
    make_variant<Tile<8, 1, 2, 2, 4, 6>>("w8_q32_k64_dma3_look6"), // dma3 + 6 operand reads ahead
    make_variant<Tile<8, 1, 4, 2, 5>>("w8_q32_k128_dma2"),        // 128-key tiles, 2-stage ring
    make_variant<Tile<8, 1, 4, 2, 5, 4>>("w8_q32_k128_dma2_look4"), // ... with 4 operand reads ahead
    make_variant<Tile<8, 1, 2, 2, 4, 0, 4>>("w8_q32_k64_dma3_pre4"),   // dma3 + 4 P.V operands read before the softmax
    make_variant<Tile<8, 1, 2, 2, 7, 0, 0>>("w8_q32_k64_dma4_pairs"),  // 4-stage ring, one barrier per 2 tiles
    make_variant<Tile<8, 1, 2, 2, 4, 0, 0, true>>("w8_q32_k64_dma3_asmcp"),   // dma3, copies as assembly
    make_variant<Tile<8, 1, 2, 2, 9, 4>>("w8_q32_k64_dma4_pingpong_look4"),   // two wave groups in opposite phases
    make_variant<Tile<8, 1, 2, 2, 4, 0, 0, false, 4>>("w8_q32_k64_dma3_asm4"),   // dma3, MFMA phases as assembly, 4 ahead
    make_variant<Tile<8, 1, 2, 2, 9, 0, 0, false, 8>>("w8_q32_k64_dma4_pingpong_asm8"),  // ... MFMA phases as assembly, 8 ahead
    make_variant<Tile<4, 1, 2, 2, 5, 4>>("w4_q32_k64_dma2_look4"),   // 4 waves, 2 workgroups per CU, 4 operand reads ahead
    make_variant<Tile<8, 1, 2, 2, 10, 0, 4>>("w8_q32_k32_dma4_thread4"),   // softmax threaded between MFMAs, 4 operands ahead
    make_variant<Tile<8, 1, 2, 2, 11, 4>>("w8_q32_k64_dma3_shift_look4"),  // waves 0-3 one phase ahead of waves 4-7
    make_roles_variant("w8_pairs32_k64_roles_ring3"),  // softmax wave + P.V wave per SIMD, P through LDS
    make_variant<Tile<8, 1, 2, 2, 4, 4, 0, false, 0, 1>>("w8_q32_k64_dma3_look4_swexp"),      // variant 11, every 2^x in software
    make_variant<Tile<8, 1, 2, 2, 4, 4, 0, false, 0, 2>>("w8_q32_k64_dma3_look4_swexp_half"), // variant 11, every other 2^x in software
    make_sched_variant("w8_q32_k64_sched_ring4"),   // hand-scheduled main loop, waves paired half a tile apart
    make_sched_persist_variant("w8_q32_k64_sched_persist"),   // ... one workgroup per CU over the items
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);
static_assert(kNumVariants == 29, "variant table");

// Measured on MI355X (same box, alternating runs): d = 128, causal or not,
// runs the hand-scheduled kernel (variant 27: headline shape 0.49-0.50 ms
// per call against 0.52-0.53 for variant 11, N = 16384 causal 1.84 against
// 1.88 ms, N = 4096 causal a tie); non-causal d = 64 runs 128-key tiles in a
// 2-stage ring with 4 operand reads ahead (variant 14); causal d = 64 runs
// 4-wave workgroups, two per CU, on a 2-stage ring of 64-key tiles (variant
// 10: twice the workgroups balance the triangular work).
constexpr int kSchedVariant = 27;
int default_variant(int bf16, int d, int causal) {
  (void)bf16;
  if (d == 128) return kSchedVariant;
  return causal ? 10 : 14;
}

// compute units of the current device (one persistent workgroup each)
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 1;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// finite test on the bit pattern (independent of floating-point compile flags)
bool finite_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof(u));
  return ((u >> 23) & 0xFFu) != 0xFFu;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Validation shared by every entry point; FA2_OK means "launch".

int check(const void* q, const void* k, const void* v, const void* o, const void* lse, int B,
          int H, int N, int d, int causal, float scale, int dtype, int variant) {
  if (dtype != FA2_DTYPE_FP16 && dtype != FA2_DTYPE_BF16) return FA2_ERR_ARG;
  if (causal != 0 && causal != 1) return FA2_ERR_ARG;
  if (!finite_bits(scale)) return FA2_ERR_ARG;
  if (variant < 0 || variant >= kNumVariants) return FA2_ERR_ARG;
  if (B < 1 || H < 1 || N < 1) return FA2_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
  if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED;
  // one head must be addressable with 32-bit byte offsets
  if ((uint64_t)N * (uint64_t)d * 2u >= (1ull << 32)) return FA2_ERR_SHAPE;
  const uint64_t bh = (uint64_t)B * (uint64_t)H;
  if (bh > (uint64_t)INT32_MAX) return FA2_ERR_SHAPE;
  const uint64_t elems = bh * (uint64_t)N * (uint64_t)d;
  if (elems >= (1ull << 62)) return FA2_ERR_SHAPE;
  // the grid must fit in one dimension for the smallest query block (128 rows)
  if (((uint64_t)N + 127) / 128 * bh > (uint64_t)INT32_MAX) return FA2_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15u)
    return FA2_ERR_ALIGN;
  const size_t tbytes = (size_t)elems * 2u;
  const size_t lbytes = (size_t)(bh * (uint64_t)N) * 4u;
  if (overlaps(o, tbytes, q, tbytes) || overlaps(o, tbytes, k, tbytes) ||
      overlaps(o, tbytes, v, tbytes) || overlaps(o, tbytes, lse, lbytes) ||
      overlaps(lse, lbytes, q, tbytes) || overlaps(lse, lbytes, k, tbytes) ||
      overlaps(lse, lbytes, v, tbytes))
    return FA2_ERR_ALIAS;
  return FA2_OK;
}

int run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
        int d, int causal, float scale, hipStream_t stream, int dtype, int variant) {
  const int st = check(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, variant);
  if (st != FA2_OK) return st;
  const uint64_t bh = (uint64_t)B * (uint64_t)H;

  const int bf16 = dtype == FA2_DTYPE_BF16;
  const int vi = variant == 0 ? default_variant(bf16, d, causal) : variant;
  const Variant& var = kVariants[vi];
  const int nqb = (N + var.rows_per_block - 1) / var.rows_per_block;
  const uint64_t blocks = (uint64_t)nqb * bh;   // <= INT32_MAX: checked for 128-row blocks

  Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = (int)bh;
  a.N = N;
  a.nqb = nqb;
  a.c = scale * 1.4426950408889634f;  // scale * log2(e)

  kernel_fn fn = var.fn[bf16][d == 128][causal];
  uint64_t grid = blocks;
  if (var.persist[bf16] && d == 128 && !causal && N % fa2::kSchedRows == 0) {
    fn = var.persist[bf16];
    grid = std::min<uint64_t>(blocks, (uint64_t)cu_count());
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(var.threads), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return FA2_ERR_LAUNCH;
  return FA2_OK;
}


// ---- backward ---------------------------------------------------------------

using fa2::BwdArgs;
using fa2::BwdTile;

typedef void (*bwd_fn)(BwdArgs);
typedef void (*delta_fn)(BwdArgs, long long);

// dK/dV kernel: 4 waves (128 keys) per workgroup, one wave per SIMD (K, V
// rows, two accumulators and two score blocks need more than 256 VGPRs).
// dQ kernel: 8 waves (256 queries) per workgroup, two waves per SIMD.
using KvTile = BwdTile<4, 1>;
using QTile = BwdTile<8, 2>;
// dQ alternative for small grids: 4 waves (128 queries) per workgroup
using QTile4 = BwdTile<4, 2>;

// dK/dV alternative: 8 waves (128 keys), two per SIMD, the dV and dK
// products split between the two waves of a SIMD.
constexpr int kSplitKeys = 128;

struct BwdKernels {
  delta_fn delta[2][2];        // [bf16][d == 128]
  bwd_fn dkdv[2][2][2];        // [bf16][d == 128][causal]
  bwd_fn dkdv_split[2][2][2];
  bwd_fn dkdv_ring[2][2][2];
  bwd_fn dkdv_ring_sub2[2][2][2];
  bwd_fn dkdv_pair[2][2][2];
  bwd_fn dkdv_pair_look[2][2][2];
  bwd_fn dkdv_pair_look2[2][2][2];
  bwd_fn dkdv_pair_look6[2][2][2];
  bwd_fn dkdv_pipe[2][2][2];
  bwd_fn dq[2][2][2];
  bwd_fn dq_ring[2][2][2];
  bwd_fn dq_look[2][2][2];
  bwd_fn dq_look2[2][2][2];
  bwd_fn dq_look6[2][2][2];
  bwd_fn dq_look_fused[2][2][2];
  bwd_fn dq_pipe[2][2][2];
  bwd_fn dq4_look[2][2];       // [bf16][causal], d = 64 only
};

template <bool BF16, int D>
constexpr void fill_bwd(BwdKernels& t) {
  t.delta[BF16][D == 128] = fa2::fa2_bwd_delta_kernel<BF16, D>;
  t.dkdv[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_kernel<BF16, D, false, KvTile>;
  t.dkdv[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_kernel<BF16, D, true, KvTile>;
  t.dkdv_split[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_split_kernel<BF16, D, false, false>;
  t.dkdv_split[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_split_kernel<BF16, D, true, false>;
  t.dkdv_ring[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_split_kernel<BF16, D, false, true>;
  t.dkdv_ring[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_split_kernel<BF16, D, true, true>;
  t.dkdv_ring_sub2[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_split_kernel<BF16, D, false, true, 2>;
  t.dkdv_ring_sub2[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_split_kernel<BF16, D, true, true, 2>;
  t.dkdv_pair[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_pair_kernel<BF16, D, false>;
  t.dkdv_pair[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_pair_kernel<BF16, D, true>;
  t.dkdv_pair_look[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_pair_kernel<BF16, D, false, 4>;
  t.dkdv_pair_look[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_pair_kernel<BF16, D, true, 4>;
  t.dkdv_pair_look2[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_pair_kernel<BF16, D, false, 2>;
  t.dkdv_pair_look2[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_pair_kernel<BF16, D, true, 2>;
  t.dkdv_pair_look6[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_pair_kernel<BF16, D, false, 6>;
  t.dkdv_pair_look6[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_pair_kernel<BF16, D, true, 6>;
  t.dkdv_pipe[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_pipe_kernel<BF16, D, false, 2>;
  t.dkdv_pipe[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_pipe_kernel<BF16, D, true, 2>;
  t.dq[BF16][D == 128][0] = fa2::fa2_bwd_dq_kernel<BF16, D, false, QTile>;
  t.dq[BF16][D == 128][1] = fa2::fa2_bwd_dq_kernel<BF16, D, true, QTile>;
  t.dq_ring[BF16][D == 128][0] = fa2::fa2_bwd_dq_kernel<BF16, D, false, QTile, true>;
  t.dq_ring[BF16][D == 128][1] = fa2::fa2_bwd_dq_kernel<BF16, D, true, QTile, true>;
  t.dq_look[BF16][D == 128][0] = fa2::fa2_bwd_dq_kernel<BF16, D, false, QTile, false, 4>;
  t.dq_look[BF16][D == 128][1] = fa2::fa2_bwd_dq_kernel<BF16, D, true, QTile, false, 4>;
  t.dq_look2[BF16][D == 128][0] = fa2::fa2_bwd_dq_kernel<BF16, D, false, QTile, false, 2>;
  t.dq_look2[BF16][D == 128][1] = fa2::fa2_bwd_dq_kernel<BF16, D, true, QTile, false, 2>;
  t.dq_look6[BF16][D == 128][0] = fa2::fa2_bwd_dq_kernel<BF16, D, false, QTile, false, 6>;
  t.dq_look6[BF16][D == 128][1] = fa2::fa2_bwd_dq_kernel<BF16, D, true, QTile, false, 6>;
  t.dq_look_fused[BF16][D == 128][0] = fa2::fa2_bwd_dq_kernel<BF16, D, false, QTile, false, 4, true>;
  t.dq_look_fused[BF16][D == 128][1] = fa2::fa2_bwd_dq_kernel<BF16, D, true, QTile, false, 4, true>;
  t.dq_pipe[BF16][D == 128][0] = fa2::fa2_bwd_dq_pipe_kernel<BF16, D, false, 4>;
  t.dq_pipe[BF16][D == 128][1] = fa2::fa2_bwd_dq_pipe_kernel<BF16, D, true, 4>;
}

BwdKernels make_bwd_kernels() {
  BwdKernels t{};
  t.dq4_look[0][0] = fa2::fa2_bwd_dq_kernel<false, 64, false, QTile4, false, 4>;
  t.dq4_look[0][1] = fa2::fa2_bwd_dq_kernel<false, 64, true, QTile4, false, 4>;
  t.dq4_look[1][0] = fa2::fa2_bwd_dq_kernel<true, 64, false, QTile4, false, 4>;
  t.dq4_look[1][1] = fa2::fa2_bwd_dq_kernel<true, 64, true, QTile4, false, 4>;
  fill_bwd<false, 64>(t);
  fill_bwd<false, 128>(t);
  fill_bwd<true, 64>(t);
  fill_bwd<true, 128>(t);
  return t;
}

const BwdKernels kBwd = make_bwd_kernels();

// backward variants: 0 = default, 1 = one-wave-per-SIMD dK/dV kernel,
// 2 = role-split dK/dV kernel, 3 = role-split with a 4-stage direct-copy
// ring; 4 and 5 = variants 3 and 1 with the dQ kernel on a 3-stage
// direct-copy ring (1-3 use the register-staged dQ kernel); 6 = variant 3
// with 64-query tiles (two 32-query sub-blocks per barrier); 7 = P handed
// from the dV wave to the dK wave of a SIMD through LDS (no S recomputed);
// 8 = variant 7 with the dQ kernel's MFMAs issued with 4 operand reads ahead;
// 9 = variant 8 with the dK/dV kernel's MFMAs ordered the same way;
// 10 = variant 9 with D computed by the dQ kernel, which runs first (two
// launches instead of three); 11 = variant 1 with 4-wave (128-query) dQ
// workgroups, MFMAs 4 operand reads ahead (at d = 128 it runs variant 1's
// dQ kernel); 12, 13 = variant 9 with 2 and 6 operand reads ahead; 14 =
// the P hand-off pipelined across query tiles (one barrier per iteration)
constexpr int kNumBwdVariants = 16;
const char* const kBwdVariantNames[kNumBwdVariants] = {"default", "dkdv_w4_occ1", "dkdv_w8_split_occ2",
                                                       "dkdv_w8_split_occ2_ring4",
                                                       "dkdv_w8_split_occ2_ring4_dq_ring3",
                                                       "dkdv_w4_occ1_dq_ring3",
                                                       "dkdv_w8_split_occ2_ring4_q64",
                                                       "dkdv_w8_pair_occ2_ring3_q64",
                                                       "dkdv_w8_pair_occ2_ring3_q64_dq_look4",
                                                       "dkdv_w8_pair_occ2_ring3_q64_look4_dq_look4",
                                                       "dkdv_w8_pair_occ2_ring3_q64_look4_dq_look4_fused_d",
                                                       "dkdv_w4_occ1_dq_w4_look4",
                                                       "dkdv_w8_pair_occ2_ring3_q64_look2_dq_look2",
                                                       "dkdv_w8_pair_occ2_ring3_q64_look6_dq_look6",
                                                       "dkdv_w8_pipe_occ2_ring3_q64_look2_dq_look4",
                                                       "dkdv_w8_pipe_occ2_ring3_q64_look2_dq_pipe_look4"};

// Measured on MI355X (bench.py --backward, alternating runs on one box): at
// d = 128 the P hand-off between the two waves of a SIMD pipelined across
// query tiles is fastest (headline shape 2.23-2.24 ms per call against
// 2.35-2.40 for the unpipelined hand-off with the same operand order,
// N = 16384 causal 8.5-8.6 against 9.4 ms; earlier steps: 2.41-2.42 without
// the operand order, 2.42-2.45 for the role split with 64-query tiles, 2.71
// with 32-query tiles and 2.95 for variant 1); at d = 64 variant 1 (0.125-0.129 ms
// against 0.130-0.133 for variants 6, 7 and 11), and for causal d = 64
// variant 11, whose 4-wave dQ workgroups balance the triangular work
// (0.095 against 0.103 ms).
int default_bwd_variant(int d, int causal) {
  if (d == 128) return 14;
  return causal ? 11 : 1;
}

int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* lse,
              const void* dout, const void* dq, const void* dk, const void* dv, const void* delta,
              int B, int H, int N, int d, int causal, float scale, int dtype, int variant) {
  if (dtype != FA2_DTYPE_FP16 && dtype != FA2_DTYPE_BF16) return FA2_ERR_ARG;
  if (variant < 0 || variant >= kNumBwdVariants) return FA2_ERR_ARG;
  if (causal != 0 && causal != 1) return FA2_ERR_ARG;
  if (!finite_bits(scale)) return FA2_ERR_ARG;
  if (B < 1 || H < 1 || N < 1) return FA2_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return FA2_ERR_NULL;
  if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED;
  if ((uint64_t)N * (uint64_t)d * 2u >= (1ull << 32)) return FA2_ERR_SHAPE;
  const uint64_t bh = (uint64_t)B * (uint64_t)H;
  if (bh > (uint64_t)INT32_MAX) return FA2_ERR_SHAPE;
  const uint64_t elems = bh * (uint64_t)N * (uint64_t)d;
  if (elems >= (1ull << 62)) return FA2_ERR_SHAPE;
  // grids: 128-key blocks, and the D kernel's 256-lane blocks of 8 elements per lane
  if (((uint64_t)N + 127) / 128 * bh > (uint64_t)INT32_MAX) return FA2_ERR_SHAPE;
  if ((elems / 8 + 255) / 256 > (uint64_t)INT32_MAX) return FA2_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse | (uintptr_t)dout |
       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)delta) & 15u)
    return FA2_ERR_ALIGN;
  const size_t tb = (size_t)elems * 2u;
  const size_t lb = (size_t)(bh * (uint64_t)N) * 4u;
  const void* in[6] = {q, k, v, o, lse, dout};
  const size_t inb[6] = {tb, tb, tb, tb, lb, tb};
  const void* out[4] = {dq, dk, dv, delta};
  const size_t outb[4] = {tb, tb, tb, lb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], outb[i], in[j], inb[j])) return FA2_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], outb[i], out[j], outb[j])) return FA2_ERR_ALIAS;
  }
  return FA2_OK;
}

int run_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int N, int d,
            int causal, float scale, hipStream_t stream, int dtype, int variant) {
  const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, causal, scale, dtype, variant);
  if (st != FA2_OK) return st;
  const uint64_t bh = (uint64_t)B * (uint64_t)H;
  const int bf16 = dtype == FA2_DTYPE_BF16;
  const int big = d == 128;

  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.BH = (int)bh;
  a.N = N;
  a.c = scale * 1.4426950408889634f;
  a.scale = scale;

  const int vi = variant == 0 ? default_bwd_variant(d, causal) : variant;
  const bool fused_d = vi == 10;
  auto launch_dq = [&]() {
    if (vi == 11 && !big) {
      a.nblk = (N + QTile4::BR - 1) / QTile4::BR;
      hipLaunchKernelGGL(kBwd.dq4_look[bf16][causal], dim3((unsigned)((uint64_t)a.nblk * bh)),
                         dim3(QTile4::THREADS), 0, stream, a);
      return hipGetLastError() == hipSuccess;
    }
    a.nblk = (N + QTile::BR - 1) / QTile::BR;
    bwd_fn dqfn = (vi == 4 || vi == 5) ? kBwd.dq_ring[bf16][big][causal]
                 : (vi == 8 || vi == 9 || vi == 14) ? kBwd.dq_look[bf16][big][causal]
                 : vi == 10             ? kBwd.dq_look_fused[bf16][big][causal]
                 : vi == 12             ? kBwd.dq_look2[bf16][big][causal]
                 : vi == 13             ? kBwd.dq_look6[bf16][big][causal]
                 : vi == 15             ? kBwd.dq_pipe[bf16][big][causal]
                                        : kBwd.dq[bf16][big][causal];
    hipLaunchKernelGGL(dqfn, dim3((unsigned)((uint64_t)a.nblk * bh)), dim3(QTile::THREADS), 0, stream, a);
    return hipGetLastError() == hipSuccess;
  };

  if (fused_d) {
    // dQ first: it computes D, uses it and writes it for the dK/dV kernel
    if (!launch_dq()) return FA2_ERR_LAUNCH;
  } else {
    // D = rowsum(dO * O): one lane per 8 elements
    const long long rows = (long long)(bh * (uint64_t)N);
    const uint64_t lanes = (uint64_t)rows * (uint64_t)(d / 8);
    a.nblk = 0;
    hipLaunchKernelGGL(kBwd.delta[bf16][big], dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, stream, a, rows);
    if (hipGetLastError() != hipSuccess) return FA2_ERR_LAUNCH;
  }

  if (vi == 2 || vi == 3 || vi == 4 || vi == 6 || vi == 7 || vi == 8 || vi == 9 || vi == 10 || vi == 12 ||
      vi == 13 || vi == 14 || vi == 15) {
    a.nblk = (N + kSplitKeys - 1) / kSplitKeys;
    bwd_fn fn = vi == 2 ? kBwd.dkdv_split[bf16][big][causal]
              : vi == 6 ? kBwd.dkdv_ring_sub2[bf16][big][causal]
              : (vi == 7 || vi == 8) ? kBwd.dkdv_pair[bf16][big][causal]
              : (vi == 9 || vi == 10) ? kBwd.dkdv_pair_look[bf16][big][causal]
              : vi == 12 ? kBwd.dkdv_pair_look2[bf16][big][causal]
              : vi == 13 ? kBwd.dkdv_pair_look6[bf16][big][causal]
              : (vi == 14 || vi == 15) ? kBwd.dkdv_pipe[bf16][big][causal]
                        : kBwd.dkdv_ring[bf16][big][causal];
    hipLaunchKernelGGL(fn, dim3((unsigned)((uint64_t)a.nblk * bh)), dim3(512), 0, stream, a);
  } else {
    a.nblk = (N + KvTile::BR - 1) / KvTile::BR;
    hipLaunchKernelGGL(kBwd.dkdv[bf16][big][causal], dim3((unsigned)((uint64_t)a.nblk * bh)),
                       dim3(KvTile::THREADS), 0, stream, a);
  }
  if (hipGetLastError() != hipSuccess) return FA2_ERR_LAUNCH;

  if (!fused_d && !launch_dq()) return FA2_ERR_LAUNCH;
  return FA2_OK;
}

}  // namespace

FA2_EXPORT int fa2_fwd_fp16(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int N, int d, int causal, float scale,
                            hipStream_t stream) {
  return run(q, k, v, o, lse, B, H, N, d, causal, scale, stream, FA2_DTYPE_FP16, 0);
}

FA2_EXPORT int fa2_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int N, int d, int causal, float scale,
                            hipStream_t stream) {
  return run(q, k, v, o, lse, B, H, N, d, causal, scale, stream, FA2_DTYPE_BF16, 0);
}

FA2_EXPORT int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int N, int d, int causal, float scale, hipStream_t stream,
                       int dtype) {
  return run(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype, 0);
}

FA2_EXPORT int fa2_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int N, int d, int causal, float scale,
                               hipStream_t stream, int dtype, int variant) {
  return run(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype, variant);
}

FA2_EXPORT int fa2_fwd_check(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, int B, int H, int N, int d, int causal,
                             float scale, int dtype, int variant) {
  return check(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, variant);
}

FA2_EXPORT int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H,
                       int N, int d, int causal, float scale, hipStream_t stream, int dtype) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, causal, scale, stream, dtype, 0);
}

FA2_EXPORT int fa2_bwd_variant(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               float* delta, int B, int H, int N, int d, int causal, float scale,
                               hipStream_t stream, int dtype, int variant) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, causal, scale, stream, dtype,
                 variant);
}

FA2_EXPORT int fa2_bwd_num_variants(void) { return kNumBwdVariants; }

FA2_EXPORT const char* fa2_bwd_variant_name(int variant) {
  if (variant < 0 || variant >= kNumBwdVariants) return nullptr;
  return kBwdVariantNames[variant];
}

FA2_EXPORT int fa2_bwd_fp16(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            float* delta, int B, int H, int N, int d, int causal, float scale,
                            hipStream_t stream) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, causal, scale, stream,
                 FA2_DTYPE_FP16, 0);
}

FA2_EXPORT int fa2_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            float* delta, int B, int H, int N, int d, int causal, float scale,
                            hipStream_t stream) {
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, causal, scale, stream,
                 FA2_DTYPE_BF16, 0);
}

FA2_EXPORT int fa2_bwd_check(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, const void* dq, const void* dk,
                             const void* dv, const float* delta, int B, int H, int N, int d,
                             int causal, float scale, int dtype) {
  return check_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, causal, scale, dtype, 0);
}

FA2_EXPORT int fa2_default_variant(int dtype, int d, int causal) {
  if (dtype != FA2_DTYPE_FP16 && dtype != FA2_DTYPE_BF16) return FA2_ERR_ARG;
  if (causal != 0 && causal != 1) return FA2_ERR_ARG;
  if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED;
  return default_variant(dtype == FA2_DTYPE_BF16, d, causal);
}

FA2_EXPORT int fa2_num_variants(void) { return kNumVariants; }

FA2_EXPORT const char* fa2_variant_name(int variant) {
  if (variant < 0 || variant >= kNumVariants) return nullptr;
  return kVariants[variant].name;
}

FA2_EXPORT const char* fa2_status_string(int status) {
  switch (status) {
    case FA2_OK: return "ok";
    case FA2_ERR_NULL: return "a tensor pointer is NULL";
    case FA2_ERR_SHAPE: return "invalid shape: B, H, N must be >= 0 and one head below 4 GiB";
    case FA2_ERR_UNSUPPORTED: return "unsupported head dimension: d must be 64 or 128";
    case FA2_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA2_ERR_ARG: return "invalid argument: scale, causal, dtype or variant";
    case FA2_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA2_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

FA2_EXPORT int fa2_version(void) { return 100; }
