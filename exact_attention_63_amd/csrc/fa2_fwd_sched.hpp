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
// (O = acc / l, LSE) is shared.  A persistent form (one workgroup per CU over
// a list of items) chains the loops of consecutive items: the last intervals
// of one item copy the next item's first tiles and load its Q.
//
// The block binds every value it reads or writes to fixed registers: Q
// fragments v[0:31], O^T accumulators v[32:95], m v178, l v179, K fragment
// addresses v[160:167], V^T fragment addresses v[168:175], copy offsets
// v[176:177], Q lane offset v185; K and V buffer descriptors s[40:43],
// s[44:47], c s48, tile count s49, this wave's LDS copy address s52, the next
// item's K, V, Q descriptors s[56:59], s[60:63], s[64:67], its Q block offset
// s68 and whether there is one s69, the tile shift past the last full tile
// s72 and the whole tiles the copies may fetch s73.  It clobbers v[96:159],
// v[180:FA2_SCHED_REG_END) but v185, a few SGPRs, m0, vcc and scc.
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
__device__ __forceinline__ u32x2 lds_tr16_at(uint32_t addr) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

// The next work item of a persistent workgroup, as the loop reads it: its K,
// V and Q buffer descriptors, the byte offset of the wave's 32 rows of its
// query block, and whether there is one (0: the loop does no prefetch).
struct SchedNext {
  __amdgpu_buffer_rsrc_t k, v, q;
  uint32_t qoff;
  uint32_t has;
};

// Per-wave values every item of a workgroup shares.
struct SchedWave {
  u32x2 dsrc;      // byte offsets (inside a tile) of this lane's two copy chunks
  u32x8 ka, va;    // LDS addresses of the K fragments and V^T fragments
  uint32_t qoff;   // this lane's byte offset inside the wave's 32 Q rows
  uint32_t m0b;    // LDS address of the wave's 2 KiB share of a tile
  uint32_t lds0;   // LDS address of the ring
};

__device__ __forceinline__ SchedWave sched_wave(uint8_t* smem, int wave, int lane) {
  constexpr int D = 128, KROW = 2 * D, DK = D / 16, DB = D / 32, VOFF = 4 * 64 * KROW;
  const int lr = lane & 31, lh = lane >> 5;
  SchedWave w;
  // the LDS chunk p of row r holds the row's logical chunk p ^ chunk_swizzle(r)
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row = (2 * wave + k) * 4 + (lane >> 4);
    w.dsrc[k] = (uint32_t)(row * KROW + 16 * ((lane & 15) ^ chunk_swizzle<D>(row)));
  }
  w.lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // K fragment of d step dk: row lr of a 32-key block, chunk 2 dk + lh
  const int kfb = lr * KROW + 16 * (lh ^ chunk_swizzle<D>(lr));
  // V^T fragments through the transpose read: lane (4e + c) of 16-lane group g
  // addresses key row 4 (g/2) + e (+8 for the high half), columns
  // 32 db + 16 (g%2) + 4c
  const int vgq = lane >> 4, ve = (lane >> 2) & 3, vc = lane & 3;
  const int vfb = (4 * (vgq >> 1) + ve) * KROW + 8 * (vc & 1) + 64 * ve +
                  16 * ((2 * (vgq & 1) | (vc >> 1)) ^ (vgq >> 1));
#pragma unroll
  for (int dk = 0; dk < DK; ++dk) w.ka[dk] = w.lds0 + (uint32_t)(kfb ^ (32 * dk));
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    w.va[2 * db] = w.lds0 + (uint32_t)(VOFF + (vfb ^ (64 * db)));
    w.va[2 * db + 1] = w.lds0 + (uint32_t)(VOFF + 8 * KROW + (vfb ^ (64 * db) ^ 32));
  }
  w.qoff = (uint32_t)(lr * KROW + 16 * lh);
  w.m0b = __builtin_amdgcn_readfirstlane(w.lds0 + (uint32_t)wave * 2048u);
  return w;
}

// Copies this wave's parts of K of tiles 0-2 and V of tiles 0-1 to ring
// stages 0-2 (inside the loop, interval j copies K of tile j+3 and V of tile
// j+2).
__device__ __forceinline__ void sched_first_copies(uint8_t* smem, const SchedWave& w, int wave,
                                                   __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                                   int nfull) {
  constexpr int TSZ = 64 * 256, VOFF = 4 * TSZ;
  for (int t = 0; t < 3 && t < nfull; ++t)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      lds_dma16(kr, smem + t * TSZ + (2 * wave + k) * 1024, w.dsrc[k], t * TSZ);
      if (t < 2) lds_dma16(vr, smem + VOFF + t * TSZ + (2 * wave + k) * 1024, w.dsrc[k], t * TSZ);
    }
}

// The wave's Q fragments of rows q_w .. q_w + 31 (rows past the buffer read
// as 0); fragment dk is q32[4 dk .. 4 dk + 3], the B operand of S^T = K Q^T.
__device__ __forceinline__ u32x32 sched_load_q(__amdgpu_buffer_rsrc_t qr, const SchedWave& w, int q_w) {
  u32x32 q32;
#pragma unroll
  for (int dk = 0; dk < 8; ++dk) {
    const u32x4 f = __builtin_amdgcn_raw_buffer_load_b128(qr, w.qoff + (uint32_t)(q_w * 256 + 32 * dk), 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) q32[4 * dk + i] = f[i];
  }
  return q32;
}

// The assembly main loop over the item's full tiles (ntiles >= 1).  Before
// the first item, K tiles 0-2 and V tiles 0-1 are in ring stages 0-2 and
// the workgroup has synchronised after every wave waited for its copies.
// With nx.has != 0 the loop leaves the next item's tiles there (the next
// loop's barriers publish them), its Q fragments in q32 and its K and V
// descriptors in kr and vr (nsub = ntv = ntiles); without, nx holds the
// current descriptors, nsub = 0 and ntv is the number of whole tiles of the
// head: the loop's last copies leave K(t) for 3 <= t <= ntiles + 2 and V(t)
// for 2 <= t <= ntiles + 1 with t < ntv in ring stage t % 4, and every copy
// has landed when it returns.
template <bool BF16>
__device__ __forceinline__ void sched_loop(f32x16& acc0, f32x16& acc1, f32x16& acc2, f32x16& acc3, float& m_run,
                                           float& l_run, u32x32& q32, __amdgpu_buffer_rsrc_t& kr,
                                           __amdgpu_buffer_rsrc_t& vr, const SchedWave& w, float c, int ntiles,
                                           const SchedNext& nx, int nsub, int ntv) {
#define FA2_SCHED_OPERANDS                                                                                 \
  : "+{v[32:47]}"(acc0), "+{v[48:63]}"(acc1), "+{v[64:79]}"(acc2), "+{v[80:95]}"(acc3), "={v178}"(m_run), \
    "={v179}"(l_run), "+{v[0:31]}"(q32), "+{s[40:43]}"(kr), "+{s[44:47]}"(vr)                              \
  : "{v[160:167]}"(w.ka), "{v[168:175]}"(w.va), "{v[176:177]}"(w.dsrc), "{v185}"(w.qoff), "{s48}"(c),     \
    "{s49}"(ntiles), "{s52}"(w.m0b), "{s[56:59]}"(nx.k), "{s[60:63]}"(nx.v), "{s[64:67]}"(nx.q),           \
    "{s68}"(nx.qoff), "{s69}"(nx.has), "{s72}"(nsub), "{s73}"(ntv)                                      \
  : FA2_SCHED_CLOBBERS
  if constexpr (BF16) asm volatile(FA2_SCHED_BF16 FA2_SCHED_OPERANDS);
  else asm volatile(FA2_SCHED_F16 FA2_SCHED_OPERANDS);
#undef FA2_SCHED_OPERANDS
}

// O = acc / l and LSE = (m + log2 l) ln 2 of the wave's rows q_w .. q_w + 31
// (stores past the buffer are dropped); O through the wave's 4 KiB of LDS at
// stage (store_o128_staged).
template <bool BF16>
__device__ __forceinline__ void sched_store(const Args& a, int bh, int q_w, int lane, const f32x16& acc0,
                                            const f32x16& acc1, const f32x16& acc2, const f32x16& acc3,
                                            float m_run, float l_run, uint8_t* stage) {
  constexpr int D = 128;
  const int N = a.N, lr = lane & 31, lh = lane >> 5;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const __amdgpu_buffer_rsrc_t orr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((uint16_t*)a.o + head_off), 0, (uint32_t)N * D * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t lsr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.lse + (size_t)bh * N), 0, (uint32_t)N * 4, kBufferWord3);
  const float l = sum_halves(l_run);
  const float inv = __builtin_amdgcn_rcpf(l);   // l >= 1: the row's largest p is 1
  store_o128_staged<BF16>(orr, q_w, lane, acc0, acc1, acc2, acc3, inv, stage);
  if (lh == 0) {
    const float lse = (m_run + log2f(l)) * 0.69314718055994530942f;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), lsr, (uint32_t)((q_w + lr) * 4), 0, 0);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sched_head(const void* base, int bh, int N) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)base + (size_t)bh * (size_t)N * 128), 0,
                                           (uint32_t)N * 256, kBufferWord3);
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
  __shared__ __attribute__((aligned(4096))) uint8_t ostage[8 * kStageBytes];   // output staging

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
      causal_item(i, a.BH, a.nqb, bh, qblk);
    }
  }
  const int N = a.N;
  const __amdgpu_buffer_rsrc_t qr = sched_head(a.q, bh, N);
  __amdgpu_buffer_rsrc_t kr = sched_head(a.k, bh, N);
  __amdgpu_buffer_rsrc_t vr = sched_head(a.v, bh, N);

  const int q_wg = qblk * BR;
  const int q_w = q_wg + wave * 32;

  // key tiles visited, and the leading ones no row of the workgroup masks
  int nt = (N + BC - 1) / BC;
  int nfull = N / BC;
  if constexpr (CAUSAL) {
    nt = min(nt, (min(q_wg + BR, N) - 1) / BC + 1);
    nfull = min(nfull, q_wg / BC);
  }

  // the first K/V copies go out before the Q loads, so that their latencies
  // overlap; the loop's first barrier publishes them
  const SchedWave w = sched_wave(smem, wave, lane);
  sched_first_copies(smem, w, wave, kr, vr, nfull);
  u32x32 q32 = sched_load_q(qr, w, q_w);
  // negative scale folded into Q (c*s = (-c)*(-s) exactly), so c >= 0 below
  const bool c_neg = a.c < 0.f;
  const float c = c_neg ? -a.c : a.c;
  if (c_neg) q32 ^= 0x80008000u;
  auto qfrag = [&](int dk) { return u32x4{q32[4 * dk], q32[4 * dk + 1], q32[4 * dk + 2], q32[4 * dk + 3]}; };

  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  float m_run = -INFINITY, l_run = 0.f;

  const int ntv = N / BC;   // whole tiles of the head
  if (nfull > 0) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    const SchedNext none{kr, vr, qr, 0u, 0u};
    sched_loop<BF16>(acc0, acc1, acc2, acc3, m_run, l_run, q32, kr, vr, w, c, nfull, none, 0, ntv);
  }

  // ---- tiles that need a mask: diagonal (causal) or past N (ragged) --------
  // At most 4 (a 256-row block crosses the diagonal in 4 tiles; a ragged
  // sequence ends in one), so tile j owns ring stage j % 4.  The loop's last
  // copies fetched K(j) for 3 <= j <= nfull + 2 and V(j) for 2 <= j <= nfull + 1
  // where j is a whole tile; the rest are copied here, before one barrier.
  if (nfull < nt) {
    __syncthreads();   // the loop's last P.V reads finished in every wave
    for (int j = nfull; j < nt; ++j) {
      const bool k_have = nfull > 0 && j >= 3 && j <= nfull + 2 && j < ntv;
      const bool v_have = nfull > 0 && j >= 2 && j <= nfull + 1 && j < ntv;
      const int st = (j % NS) * TSZ;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (!k_have) lds_dma16(kr, smem + st + (2 * wave + k) * 1024, w.dsrc[k], j * TSZ);
        if (!v_have) lds_dma16(vr, smem + VOFF + st + (2 * wave + k) * 1024, w.dsrc[k], j * TSZ);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    for (int j = nfull; j < nt; ++j) {
      const int key0 = j * BC;
      if (CAUSAL && key0 > q_w + 31) continue;     // above this wave's diagonal
      const uint32_t st = (uint32_t)((j % NS) * TSZ);
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int dk = 0; dk < DK; ++dk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 kf = lds_load_b128(w.ka[dk] + st + kb * 32 * KROW);
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
        for (int h = 0; h < 2; ++h) {
          float p[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            p[t] = __builtin_amdgcn_exp2f(s[kb][8 * h + t] - m_use);
            rs += p[t];
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) pf[kb][h][t] = E::pack(p[2 * t], p[2 * t + 1]);
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
          for (int h = 0; h < 2; ++h) {
            const int roff = (32 * kb + 16 * h) * KROW;
            const u32x2 lo = lds_tr16_at(w.va[2 * db] + st + roff);
            const u32x2 hi = lds_tr16_at(w.va[2 * db + 1] + st + roff);
            acc = E::mfma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kb][h], acc);
          }
      }
    }
  }

  sched_store<BF16>(a, bh, q_w, lane, acc0, acc1, acc2, acc3, m_run, l_run, ostage + wave * kStageBytes);
}

// Persistent form for sequences of whole query blocks (N % 256 == 0), no
// mask: a grid of one workgroup per CU walks the (head, query block) items,
// and the loop of each item prefetches the next one's first K/V tiles and Q
// in its last intervals, so that neither the copies' latency nor the
// workgroup start-up falls between items.  Workgroup b runs on XCD b % 8
// (dispatch is round robin over the 8 XCDs); the items are cut into 8
// consecutive ranges, one per XCD, so that the workgroups that read one
// head's K and V share an L2.
template <bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fa2_fwd_sched_persist_kernel(Args a) {
  constexpr int BR = kSchedRows, NS = 4, TSZ = 64 * 256;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * NS * TSZ];
  __shared__ __attribute__((aligned(4096))) uint8_t ostage[8 * kStageBytes];   // output staging

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int N = a.N, nqb = a.nqb;
  const int ntiles = N / 64;

  const int total = nqb * a.BH, G = gridDim.x, b = blockIdx.x;
  const bool by_xcd = total % 8 == 0 && G % 8 == 0;
  const int per_x = total / 8, gx = G / 8;
  // the workgroup's i-th item, or -1
  auto item = [&](int i) -> int {
    if (by_xcd) {
      const int r = i * gx + b / 8;
      return r < per_x ? (b % 8) * per_x + r : -1;
    }
    const int r = b + i * G;
    return r < total ? r : -1;
  };

  int cur = item(0);
  if (cur < 0) return;
  const SchedWave w = sched_wave(smem, wave, lane);
  int bh = cur / nqb, qblk = cur % nqb;
  __amdgpu_buffer_rsrc_t kr = sched_head(a.k, bh, N);
  __amdgpu_buffer_rsrc_t vr = sched_head(a.v, bh, N);
  sched_first_copies(smem, w, wave, kr, vr, ntiles);
  u32x32 q32 = sched_load_q(sched_head(a.q, bh, N), w, qblk * BR + wave * 32);
  const bool c_neg = a.c < 0.f;
  const float c = c_neg ? -a.c : a.c;
  if (c_neg) q32 ^= 0x80008000u;
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  for (int i = 1;; ++i) {
    const int nxt = item(i);
    SchedNext nx;
    if (nxt >= 0) {
      const int nbh = nxt / nqb;
      nx = SchedNext{sched_head(a.k, nbh, N), sched_head(a.v, nbh, N), sched_head(a.q, nbh, N),
                     (uint32_t)(((nxt % nqb) * BR + wave * 32) * 256), 1u};
    } else {
      nx = SchedNext{kr, vr, kr, 0u, 0u};
    }
    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    float m_run, l_run;
    sched_loop<BF16>(acc0, acc1, acc2, acc3, m_run, l_run, q32, kr, vr, w, c, ntiles, nx, ntiles, ntiles);
    sched_store<BF16>(a, bh, qblk * BR + wave * 32, lane, acc0, acc1, acc2, acc3, m_run, l_run,
                      ostage + wave * kStageBytes);
    if (nxt < 0) break;
    bh = nxt / nqb;
    qblk = nxt % nqb;
    if (c_neg) q32 ^= 0x80008000u;
  }
}

}  // namespace fa2
