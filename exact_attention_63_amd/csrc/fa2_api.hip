// fa2_api.hip -- host side of the C ABI declared in include/fa2.h: argument
// validation, the tile-variant table and the kernel launch.
//
// The call enqueues one kernel and returns.  It allocates nothing (the method
// needs O(N) memory: only the inputs and outputs), keeps no state besides
// constant tables, and validates every argument before touching the HIP
// runtime, so an invalid call has no effect.
#include <stdint.h>
#include <string.h>

#include "fa2.h"
#include "fa2_fwd_kernel.hpp"

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
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

// Measured on MI355X (bench.py, same box, each variant twice, alternating):
// non-causal d = 128 is fastest with 64-key tiles in a 3-stage direct-copy
// ring and 4 operand reads ahead (variant 11); causal d = 128 and
// non-causal d = 64 with 128-key tiles in a 2-stage ring and 4 operand reads
// ahead (variant 14); causal d = 64 with 4-wave workgroups, two per CU, on a
// 2-stage ring of 64-key tiles (variant 10: twice the workgroups balance the
// triangular work, and the two workgroups of a CU are not held in step by
// one barrier).
int default_variant(int bf16, int d, int causal) {
  (void)bf16;
  if (d == 128) return causal ? 14 : 11;
  return causal ? 10 : 14;
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

// Validation shared by every entry point; FA2_OK means "launch", a positive
// kEmpty means "valid and nothing to do".
constexpr int kEmpty = 1;

int check(const void* q, const void* k, const void* v, const void* o, const void* lse, int B,
          int H, int N, int d, int causal, float scale, int dtype, int variant) {
  if (dtype != FA2_DTYPE_FP16 && dtype != FA2_DTYPE_BF16) return FA2_ERR_ARG;
  if (causal != 0 && causal != 1) return FA2_ERR_ARG;
  if (!finite_bits(scale)) return FA2_ERR_ARG;
  if (variant < 0 || variant >= kNumVariants) return FA2_ERR_ARG;
  if (B < 0 || H < 0 || N < 0) return FA2_ERR_SHAPE;
  if (B == 0 || H == 0 || N == 0) return kEmpty;
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
  if (st == kEmpty) return FA2_OK;
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
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(var.threads), 0, stream, a);
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
  const int st = check(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, variant);
  return st == kEmpty ? FA2_OK : st;
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
    case FA2_ERR_ALIAS: return "the output overlaps an input or the other output";
    case FA2_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

FA2_EXPORT int fa2_version(void) { return 100; }
