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
#include "fa2_fwd_fp8.hpp"
#include "fa2_fwd_fp8_sched.hpp"

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
  using D64 = Tile<8, 1, 4, 2, 2, 4>;
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
// default_variant() below.  Besides the defaults the table keeps the plain
// register-staged loop (the simplest form of the method), the previous d = 128
// default (the compiler-scheduled loop the hand-scheduled one replaced), the
// software-exp2 alternative and the role-split kernel.
const Variant kVariants[] = {
    {"default", 0, 0, {}, {nullptr, nullptr}},
    make_variant<Tile<4, 1, 2, 2>>("w4_q32_k64_occ2"),                // 1: register-staged 2-stage ring, 4 waves x 32 rows
    make_variant<Tile<4, 1, 2, 2, 2>>("w4_q32_k64_dma2"),             // 2: direct copies, 2 stages, two workgroups per CU
    make_variant<Tile<8, 1, 4, 2, 2, 4>>("w8_q32_k128_dma2_look4"),   // 3: 128-key tiles, 2 stages, 4 operand reads ahead
    make_variant<Tile<8, 1, 2, 2, 3, 4>>("w8_q32_k64_dma3_look4"),    // 4: 64-key tiles, 3 stages, 4 operand reads ahead
    make_variant<Tile<8, 1, 2, 2, 3, 4, 2>>("w8_q32_k64_dma3_look4_swexp_half"),  // 5: variant 4, every other 2^x in software
    make_roles_variant("w8_pairs32_k64_roles_ring3"),                 // 6: softmax wave + P.V wave per SIMD, P through LDS
    make_sched_variant("w8_q32_k64_sched_ring4"),                     // 7: hand-scheduled d = 128 loop
    make_sched_persist_variant("w8_q32_k64_sched_persist"),           // 8: ... persistent where the shape allows
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);
static_assert(kNumVariants == 9, "variant table");

// Measured on MI355X (same box, alternating runs): d = 128 runs the
// hand-scheduled loop, persistent for non-causal N % 256 == 0 (headline shape
// 0.471 ms against 0.483 for one workgroup per item and 0.52-0.53 for variant
// 4; N = 16384 causal 1.84 against 1.88 ms); d = 64 runs 128-key tiles in a
// 2-stage ring with 4 operand reads ahead (variant 3), causal too: on
// B=4, H=16, N=1024, causal, 23.5 against 25.2 us per call for the 4-wave
// workgroups of variant 2 (bench runs alternating over three rounds).
constexpr int kSchedVariant = 8;
int default_variant(int bf16, int d, int causal) {
  (void)bf16;
  (void)causal;
  if (d == 128) return kSchedVariant;
  return 3;
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


// ---- FP8 forward ------------------------------------------------------------

typedef void (*fp8_fn)(fa2::Fp8Args);
// Kernel per (d, causal).  Measured on MI355X with the configurations timed
// in turn over six rounds (medians; outputs bitwise equal across them):
// non-causal, 4-wave workgroups three per CU: 324 against 368 us for 8-wave
// workgroups (two waves per SIMD of one workgroup) on B=8, H=32, N=2048,
// d=128, and within 2 % at d = 64; causal, 8-wave workgroups: 99.6 against
// 110.4 us (4-wave, three per CU) on B=2, H=16, N=4096, d=128, and 18.4
// against 19.3 us at d = 64.
struct Fp8Kernel {
  fp8_fn fn;
  int waves;   // waves per workgroup (32 query rows each)
};
const Fp8Kernel kFp8[2][2] = {
    {{fa2::fa2_fwd_fp8_kernel<64, false, 4, 3>, 4}, {fa2::fa2_fwd_fp8_kernel<64, true, 8, 2>, 8}},
    {{fa2::fa2_fwd_fp8_kernel<128, false, 4, 3>, 4}, {fa2::fa2_fwd_fp8_kernel<128, true, 8, 2>, 8}}};
// the hand-scheduled d = 128 kernel (8 waves x 32 rows), per causal
const Fp8Kernel kFp8Sched[2] = {{fa2::fa2_fwd_fp8_sched_kernel<false>, 8}, {fa2::fa2_fwd_fp8_sched_kernel<true>, 8}};
// the smallest query block of the FP8 kernels (bounds the grid)
constexpr int kFp8MinRows = 128;
// FP8 variants: 0 = default, 1 = tile by tile (fa2_fwd_fp8_kernel), 2 = the
// scheduled loop (d = 128 only)
constexpr int kNumFp8Variants = 3;
const char* const kFp8VariantNames[kNumFp8Variants] = {"default", "tile_by_tile", "sched_ring4"};
// Measured on MI355X with the variants timed in turn (same box, medians,
// outputs bitwise equal): causal d = 128, B=2, H=16, N=4096: 86.7 us for the
// scheduled loop against 100.5 us tile by tile; non-causal B=8, H=32,
// N=2048: 329 against 315 us (the scheduled loop's start and end of every
// 256-row item cost more than the tile-by-tile kernel's three 4-wave
// workgroups per CU, which overlap theirs; at N=8192 the two are within 1 %).
int default_fp8_variant(int d, int causal) { return d == 128 && causal ? 2 : 1; }

// c = scale * descale_q * descale_k * log2(e), in double, then float
float fp8_exponent_scale(float scale, float dq, float dk) {
  return (float)((double)scale * (double)dq * (double)dk * 1.4426950408889634);
}

int check_fp8(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int H,
              int N, int d, int causal, float scale, float dq, float dk, float dv, int variant) {
  if (causal != 0 && causal != 1) return FA2_ERR_ARG;
  if (variant < 0 || variant >= kNumFp8Variants) return FA2_ERR_ARG;
  if (!finite_bits(scale) || !finite_bits(dq) || !finite_bits(dk) || !finite_bits(dv)) return FA2_ERR_ARG;
  if (!finite_bits(fp8_exponent_scale(scale, dq, dk))) return FA2_ERR_ARG;
  if (B < 1 || H < 1 || N < 1) return FA2_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
  if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED;
  if (variant == 2 && d != 128) return FA2_ERR_UNSUPPORTED;
  // one head of o (2-byte elements) must be addressable with 32-bit byte offsets
  if ((uint64_t)N * (uint64_t)d * 2u >= (1ull << 32)) return FA2_ERR_SHAPE;
  const uint64_t bh = (uint64_t)B * (uint64_t)H;
  if (bh > (uint64_t)INT32_MAX) return FA2_ERR_SHAPE;
  const uint64_t elems = bh * (uint64_t)N * (uint64_t)d;
  if (elems >= (1ull << 62)) return FA2_ERR_SHAPE;
  if (((uint64_t)N + kFp8MinRows - 1) / kFp8MinRows * bh > (uint64_t)INT32_MAX) return FA2_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15u)
    return FA2_ERR_ALIGN;
  const size_t ib = (size_t)elems;         // one byte per input element
  const size_t ob = (size_t)elems * 2u;    // bf16 output
  const size_t lb = (size_t)(bh * (uint64_t)N) * 4u;
  if (overlaps(o, ob, q, ib) || overlaps(o, ob, k, ib) || overlaps(o, ob, v, ib) || overlaps(o, ob, lse, lb) ||
      overlaps(lse, lb, q, ib) || overlaps(lse, lb, k, ib) || overlaps(lse, lb, v, ib))
    return FA2_ERR_ALIAS;
  return FA2_OK;
}

int run_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
            int causal, float scale, float dq, float dk, float dv, hipStream_t stream, int variant) {
  const int st = check_fp8(q, k, v, o, lse, B, H, N, d, causal, scale, dq, dk, dv, variant);
  if (st != FA2_OK) return st;
  const uint64_t bh = (uint64_t)B * (uint64_t)H;
  fa2::Fp8Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = (int)bh;
  a.N = N;
  const int vi = variant == 0 ? default_fp8_variant(d, causal) : variant;
  const Fp8Kernel& kern = vi == 2 ? kFp8Sched[causal] : kFp8[d == 128][causal];
  const int rows = 32 * kern.waves;
  a.nqb = (N + rows - 1) / rows;
  a.c = fp8_exponent_scale(scale, dq, dk);
  a.dv = dv;
  const uint64_t blocks = (uint64_t)a.nqb * bh;
  hipLaunchKernelGGL(kern.fn, dim3((unsigned)blocks), dim3(64 * kern.waves), 0, stream, a);
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

// dK/dV with P handed between the two waves of a SIMD: 8 waves (128 keys).
constexpr int kPairKeys = 128;

struct BwdKernels {
  delta_fn delta[2][2];        // [bf16][d == 128]
  bwd_fn dkdv[2][2][2];        // [bf16][d == 128][causal]
  bwd_fn dkdv_pair[2][2][2];   // P hand-off, 4 operand reads ahead
  bwd_fn dkdv_pipe[2][2][2];   // P hand-off pipelined across query tiles, 2 reads ahead
  bwd_fn dq[2][2][2];
  bwd_fn dq_look[2][2][2];     // 4 operand reads ahead
  bwd_fn dq4_look[2][2];       // [bf16][causal], d = 64 only
};

template <bool BF16, int D>
constexpr void fill_bwd(BwdKernels& t) {
  t.delta[BF16][D == 128] = fa2::fa2_bwd_delta_kernel<BF16, D>;
  t.dkdv[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_kernel<BF16, D, false, KvTile>;
  t.dkdv[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_kernel<BF16, D, true, KvTile>;
  t.dkdv_pair[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_pair_kernel<BF16, D, false, 4>;
  t.dkdv_pair[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_pair_kernel<BF16, D, true, 4>;
  t.dkdv_pipe[BF16][D == 128][0] = fa2::fa2_bwd_dkdv_pipe_kernel<BF16, D, false, 2>;
  t.dkdv_pipe[BF16][D == 128][1] = fa2::fa2_bwd_dkdv_pipe_kernel<BF16, D, true, 2>;
  t.dq[BF16][D == 128][0] = fa2::fa2_bwd_dq_kernel<BF16, D, false, QTile>;
  t.dq[BF16][D == 128][1] = fa2::fa2_bwd_dq_kernel<BF16, D, true, QTile>;
  t.dq_look[BF16][D == 128][0] = fa2::fa2_bwd_dq_kernel<BF16, D, false, QTile, 4>;
  t.dq_look[BF16][D == 128][1] = fa2::fa2_bwd_dq_kernel<BF16, D, true, QTile, 4>;
}

BwdKernels make_bwd_kernels() {
  BwdKernels t{};
  t.dq4_look[0][0] = fa2::fa2_bwd_dq_kernel<false, 64, false, QTile4, 4>;
  t.dq4_look[0][1] = fa2::fa2_bwd_dq_kernel<false, 64, true, QTile4, 4>;
  t.dq4_look[1][0] = fa2::fa2_bwd_dq_kernel<true, 64, false, QTile4, 4>;
  t.dq4_look[1][1] = fa2::fa2_bwd_dq_kernel<true, 64, true, QTile4, 4>;
  fill_bwd<false, 64>(t);
  fill_bwd<false, 128>(t);
  fill_bwd<true, 64>(t);
  fill_bwd<true, 128>(t);
  return t;
}

const BwdKernels kBwd = make_bwd_kernels();

// backward variants: 0 = default; 1 = one-wave-per-SIMD dK/dV kernel with the
// 8-wave dQ kernel; 2 = P handed from the dV wave to the dK wave of a SIMD
// through LDS (no S recomputed), both kernels' MFMAs issued with 4 operand
// reads ahead; 3 = variant 1 with 4-wave (128-query) dQ workgroups, 4 reads
// ahead (at d = 128 it runs variant 1's dQ kernel); 4 = the P hand-off
// pipelined across query tiles (one barrier per iteration)
constexpr int kNumBwdVariants = 5;
const char* const kBwdVariantNames[kNumBwdVariants] = {"default", "dkdv_w4_occ1",
                                                       "dkdv_w8_pair_occ2_ring3_q64_look4_dq_look4",
                                                       "dkdv_w4_occ1_dq_w4_look4",
                                                       "dkdv_w8_pipe_occ2_ring3_q64_look2_dq_look4"};

// Measured on MI355X with the variants timed in turn over five rounds
// (medians, one process): the P hand-off between the two waves of a SIMD
// pipelined across query tiles (variant 4) is fastest everywhere: headline
// shape 2.13 ms against 2.25 (variant 2) and 2.97 (variant 1); N = 4096
// causal 0.593 against 0.631 and 0.778 ms; B=4, H=16, N=1024, d=64, 98.0 us
// against 111-112 us for variants 1-3, and causal 85.7 against 88.8-96.7 us.
int default_bwd_variant(int d, int causal) {
  (void)d;
  (void)causal;
  return 4;
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

  // D = rowsum(dO * O): one lane per 8 elements
  const long long rows = (long long)(bh * (uint64_t)N);
  const uint64_t lanes = (uint64_t)rows * (uint64_t)(d / 8);
  a.nblk = 0;
  hipLaunchKernelGGL(kBwd.delta[bf16][big], dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, stream, a, rows);
  if (hipGetLastError() != hipSuccess) return FA2_ERR_LAUNCH;

  // dK, dV
  if (vi == 2 || vi == 4) {
    a.nblk = (N + kPairKeys - 1) / kPairKeys;
    bwd_fn fn = vi == 2 ? kBwd.dkdv_pair[bf16][big][causal] : kBwd.dkdv_pipe[bf16][big][causal];
    hipLaunchKernelGGL(fn, dim3((unsigned)((uint64_t)a.nblk * bh)), dim3(512), 0, stream, a);
  } else {
    a.nblk = (N + KvTile::BR - 1) / KvTile::BR;
    hipLaunchKernelGGL(kBwd.dkdv[bf16][big][causal], dim3((unsigned)((uint64_t)a.nblk * bh)),
                       dim3(KvTile::THREADS), 0, stream, a);
  }
  if (hipGetLastError() != hipSuccess) return FA2_ERR_LAUNCH;

  // dQ
  if (vi == 3 && !big) {
    a.nblk = (N + QTile4::BR - 1) / QTile4::BR;
    hipLaunchKernelGGL(kBwd.dq4_look[bf16][causal], dim3((unsigned)((uint64_t)a.nblk * bh)),
                       dim3(QTile4::THREADS), 0, stream, a);
  } else {
    a.nblk = (N + QTile::BR - 1) / QTile::BR;
    bwd_fn dqfn = (vi == 2 || vi == 4) ? kBwd.dq_look[bf16][big][causal] : kBwd.dq[bf16][big][causal];
    hipLaunchKernelGGL(dqfn, dim3((unsigned)((uint64_t)a.nblk * bh)), dim3(QTile::THREADS), 0, stream, a);
  }
  if (hipGetLastError() != hipSuccess) return FA2_ERR_LAUNCH;
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

FA2_EXPORT int fa2_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int N, int d, int causal, float scale, float descale_q, float descale_k,
                           float descale_v, hipStream_t stream) {
  return run_fp8(q, k, v, o, lse, B, H, N, d, causal, scale, descale_q, descale_k, descale_v, stream, 0);
}

FA2_EXPORT int fa2_fwd_fp8_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                   int H, int N, int d, int causal, float scale, float descale_q,
                                   float descale_k, float descale_v, hipStream_t stream, int variant) {
  return run_fp8(q, k, v, o, lse, B, H, N, d, causal, scale, descale_q, descale_k, descale_v, stream, variant);
}

FA2_EXPORT int fa2_fwd_fp8_check(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, int B, int H, int N, int d, int causal, float scale,
                                 float descale_q, float descale_k, float descale_v) {
  return check_fp8(q, k, v, o, lse, B, H, N, d, causal, scale, descale_q, descale_k, descale_v, 0);
}

FA2_EXPORT int fa2_fwd_fp8_variant_check(const void* q, const void* k, const void* v, const void* o,
                                         const float* lse, int B, int H, int N, int d, int causal,
                                         float scale, float descale_q, float descale_k, float descale_v,
                                         int variant) {
  return check_fp8(q, k, v, o, lse, B, H, N, d, causal, scale, descale_q, descale_k, descale_v, variant);
}

FA2_EXPORT int fa2_fp8_num_variants(void) { return kNumFp8Variants; }

FA2_EXPORT const char* fa2_fp8_variant_name(int variant) {
  return variant >= 0 && variant < kNumFp8Variants ? kFp8VariantNames[variant] : nullptr;
}

FA2_EXPORT int fa2_fp8_default_variant(int d, int causal) { return default_fp8_variant(d, causal); }

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
