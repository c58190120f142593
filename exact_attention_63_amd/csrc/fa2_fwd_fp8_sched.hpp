// fa2_fwd_fp8_sched.hpp -- the scheduled FP8 (E4M3) forward kernel, d = 128.
//
// Same method, FP8 scheme and layouts as fa2_fwd_fp8.hpp ("FlashAttention v2
// better parallelism + work partitioning" diagram: grid over (batch, head,
// query block), sliced-Q over the waves, online softmax, both products on the
// FP8 matrix cores), with the loop over full key tiles written out as a
// hand-scheduled assembly block (gen_fwd_fp8_sched.py writes it):
//   * 8 waves x 32 query rows, two per SIMD; in the interval of tile j every
//     wave issues the P.V MFMAs of tile j-1 and the score MFMAs of tile j+1,
//     with the softmax of tile j spread between them (the overlap of the
//     "FlashAttention v4 Blackwell pipeline co-design" diagram's pseudo-code
//     panel, by software pipelining within each wave);
//   * 64-key tiles of 8 KiB in a 4-stage LDS ring (K and V), filled by direct
//     global->LDS copies two tiles ahead, one barrier per tile;
//   * the lazy reference (threshold 2.75, base 2) checked on the lane max of
//     the raw scores before any 2^x, with a short out-of-line update when
//     some row moves, and acc rescaled at the end of that interval.
// Tiles that need a mask (crossing the causal diagonal, or past the end of a
// ragged sequence: at most 4 per workgroup) run the plain C++ steps of
// Fp8Wave after the block, from their ring stages: the loop's last copies
// already fetched those of them that are whole tiles of the head, the rest
// are copied together before one barrier.  The epilogue is Fp8Wave::store.
//
// The block binds every value it reads or writes to fixed registers: Q
// fragments v[0:15], O^T accumulators v[16:79], K and V^T fragment addresses
// v[144:147], v[148:151], copy offset v152, m v153, l v154; K and V buffer
// descriptors s[40:43], s[44:47], c s48, full-tile count s49, this wave's
// LDS copy address s52, whole tiles of the head s60.  It clobbers v[80:143],
// v[155:FA2_FP8_SCHED_REG_END), a few SGPRs, m0, vcc and scc.
#pragma once

#include "fa2_fwd_fp8.hpp"
#include "fa2_fwd_fp8_sched.inc"

namespace fa2 {

static_assert(FA2_FP8_SCHED_R_Q == 0 && FA2_FP8_SCHED_R_ACC == 16 && FA2_FP8_SCHED_R_KA == 144 &&
                  FA2_FP8_SCHED_R_VA == 148 && FA2_FP8_SCHED_R_DSRC == 152 && FA2_FP8_SCHED_R_M == 153 &&
                  FA2_FP8_SCHED_R_L == 154,
              "register bindings of fp8_sched_loop follow the generator");
static_assert(FA2_FP8_SCHED_S_KDESC == 40 && FA2_FP8_SCHED_S_VDESC == 44 && FA2_FP8_SCHED_S_C == 48 &&
                  FA2_FP8_SCHED_S_T == 49 && FA2_FP8_SCHED_S_M0B == 52 && FA2_FP8_SCHED_S_NTV == 60,
              "SGPR bindings of fp8_sched_loop follow the generator");
static_assert(FA2_FP8_SCHED_REG_END <= 240, "the loop leaves VGPRs for the compiler");

// Workgroups of the scheduled FP8 kernel cover 256 query rows.
constexpr int kFp8SchedRows = 256;

// The assembly loop over the ntiles >= 1 full tiles of the wave's head (ntv:
// whole 64-key tiles in the head, ntv >= ntiles).  Before it, K tiles 0-2 and
// V tiles 0-1 (those below ntiles) are in ring stages 0-2 and the workgroup
// has synchronised after every wave waited for its copies; when it returns,
// every copy it issued has landed, K(t) for 3 <= t <= ntiles + 2 and V(t) for
// 2 <= t <= ntiles + 1 with t < ntv in ring stage t % 4.
__device__ __forceinline__ void fp8_sched_loop(f32x16& acc0, f32x16& acc1, f32x16& acc2, f32x16& acc3,
                                               float& m_run, float& l_run, const i32x8& q0, const i32x8& q1,
                                               __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, u32x4 ka,
                                               u32x4 va, uint32_t dsrc, float c, int ntiles, uint32_t m0b,
                                               int ntv) {
  asm volatile(FA2_FP8_SCHED
               : "+{v[16:31]}"(acc0), "+{v[32:47]}"(acc1), "+{v[48:63]}"(acc2), "+{v[64:79]}"(acc3),
                 "={v153}"(m_run), "={v154}"(l_run)
               : "{v[0:7]}"(q0), "{v[8:15]}"(q1), "{v[144:147]}"(ka), "{v[148:151]}"(va), "{v152}"(dsrc),
                 "{s[40:43]}"(kr), "{s[44:47]}"(vr), "{s48}"(c), "{s49}"(ntiles), "{s52}"(m0b), "{s60}"(ntv)
               : FA2_FP8_SCHED_CLOBBERS);
}

template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fa2_fwd_fp8_sched_kernel(Fp8Args a) {
  constexpr int D = 128, NW = 8, NS = 4;
  using G = Fp8Geom<D, NW>;
  constexpr int TSZ = G::TSZ;
  static_assert(G::CPW == 1 && G::BC == 64 && G::BR == kFp8SchedRows, "the loop's geometry");
  __shared__ __attribute__((aligned(4096))) uint8_t smem[2 * NS * TSZ];   // K stages, then V stages
  static_assert(NW * kStageBytes <= 2 * NS * TSZ, "the ring holds the output staging");

  Fp8Wave<D, CAUSAL, NW> w;
  w.init(a, smem);
  const int nt = w.nt;
  const int ntv = w.N / G::BC;                   // whole tiles of the head
  int nfull = ntv;                               // leading tiles no row of the workgroup masks
  if constexpr (CAUSAL) nfull = min(nfull, w.q_wg / G::BC);

  // K of tiles 0-2 and V of tiles 0-1 (the loop copies K(j+3) and V(j+2) in
  // interval j); the Q loads were issued before, so this waits for both
  for (int t = 0; t < 3 && t < nfull; ++t) {
    w.copy(w.kr, t, t * TSZ);
    if (t < 2) w.copy(w.vr, t, (NS + t) * TSZ);
  }
  FA2_WAIT_VMCNT(0);
  __syncthreads();

  if (nfull > 0) {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    const u32x4 ka = {lds0 + (uint32_t)w.ka[0], lds0 + (uint32_t)w.ka[1], lds0 + (uint32_t)(w.ka[0] ^ 64),
                      lds0 + (uint32_t)(w.ka[1] ^ 64)};
    const u32x4 va = {lds0 + (uint32_t)w.vb, lds0 + (uint32_t)(w.vb ^ 32), lds0 + (uint32_t)(w.vb ^ 64),
                      lds0 + (uint32_t)(w.vb ^ 96)};
    fp8_sched_loop(w.acc[0], w.acc[1], w.acc[2], w.acc[3], w.m_run, w.l_run, w.qf[0], w.qf[1], w.kr, w.vr, ka, va,
                   w.dsrc[0], w.c, nfull, w.ldsw, ntv);
  }

  // ---- tiles that need a mask: diagonal (causal) or past N (ragged) --------
  // At most 4 (a 256-row block crosses the diagonal in 4 tiles; a ragged
  // sequence ends in one), so tile j owns ring stage j % 4.
  if (nfull < nt) {
    __syncthreads();   // the loop's last P.V reads finished in every wave
    for (int j = nfull; j < nt; ++j) {
      const bool k_have = nfull > 0 && j >= 3 && j <= nfull + 2 && j < ntv;
      const bool v_have = nfull > 0 && j >= 2 && j <= nfull + 1 && j < ntv;
      if (!k_have) w.copy(w.kr, j, (j % NS) * TSZ);
      if (!v_have) w.copy(w.vr, j, (NS + j % NS) * TSZ);
    }
    FA2_WAIT_VMCNT(0);
    __syncthreads();
    for (int j = nfull; j < nt; ++j) {
      const int key0 = j * G::BC;
      if (CAUSAL && key0 > w.q_w + 31) continue;     // above this wave's diagonal
      f32x16 sc[G::KB];
      i32x8 pk[G::PS];
      float alpha;
      w.scores(smem + (j % NS) * TSZ, sc);
      if (w.masked(key0)) w.template softmax<true>(sc, key0, pk, alpha);
      else w.template softmax<false>(sc, key0, pk, alpha);
      w.rescale(alpha);
      w.pv(smem + (NS + j % NS) * TSZ, pk);
    }
  }
  __syncthreads();   // every wave is done with the ring: it stages the output
  w.store(a, smem + (threadIdx.x >> 6) * kStageBytes);
}

}  // namespace fa2
