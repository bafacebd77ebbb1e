// qmm_slab.hip -- the slab kernels for 17..64 activation rows (activations
// streamed through an LDS ring by loader waves), unsplit and split along K.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qmm_device.h"

namespace qmm {

// ---------------------------------------------------------------------------
// Slab kernel for 17..64 activation rows.  One workgroup per compute unit
// owning TM tiles of W; K is walked in NS slices of four chunks (512 k).
//   * four loader waves copy activation slices straight from global memory
//     into a ring of RB LDS slots (LDS-direct loads: no registers), running
//     up to RB-1 slices ahead; they wait only on their own loads;
//   * 4*TM compute waves: wave (i, kp) owns tile slot i and chunk kp of every
//     slice, keeps its weight loads DR slices ahead in a register ring, and
//     forms the per-group activation sums with an all-ones MFMA;
//   * one barrier per slice; the slice loop is unrolled, so every wait on
//     memory is an exact count and no wave waits on another's loads.
// An LDS slot holds [16*MT rows][64 vectors of 16 bytes]; row m keeps its
// vector v at v ^ (m & 15) (16 rows reading one column hit distinct banks).
// Rows >= M repeat row M-1 (their outputs are never stored).  The four
// partial tiles of each tile are added through LDS in K order at the end.
// ---------------------------------------------------------------------------
template <int BITS, int MT, int TM, int NS, int RB, int DR, typename ST>
__global__ void __launch_bounds__((TM * 4 + 4) * 64) slab_kernel(LaunchArgs a) {
  constexpr int KP = 4, NWC = TM * KP, NWL = 4;
  constexpr int ROWS = 16 * MT;
  constexpr int SK = KP * kChunkK;  // k per slice
  constexpr int SLOT = ROWS * 64;   // vectors per slot
  constexpr int RPL = ROWS / NWL;   // rows per loader wave per slice
  constexpr int NB = RB < NS ? RB : NS;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4* xs = reinterpret_cast<u32x4*>(lds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nT = a.N / kTileN, nC = a.K / kChunkK;
  const int M = a.M;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  if (wave >= NWC) {
    // ---- loader waves
    const int lw = __builtin_amdgcn_readfirstlane(wave - NWC);  // wave-uniform
    const uint16_t* __restrict__ xg = reinterpret_cast<const uint16_t*>(a.x);
    auto issue = [&](int s) {
      u32x4* slot = xs + (s % RB) * SLOT;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const int m = lw + i * NWL;
        const int v = lane ^ (m & 15);
        const int col = min(s * SK + 8 * v, a.K - 8);
        const uint16_t* src = xg + (long)min(m, M - 1) * a.ldx + col;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)src,
            (__attribute__((address_space(3))) void*)(slot + m * 64), 16, 0, 0);
      }
    };
#pragma unroll
    for (int s = 0; s < NB; ++s) issue(s);
    wait_vm<(NB - 1) * RPL>();
    wg_barrier();
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      // after barrier j every compute wave is done with slice j-1
      if (j >= 1 && j - 1 + RB < NS) issue(j - 1 + RB);
      if (j + 1 < NS) {
        // slices issued after slice j+1 may stay in flight
        const int last = min(j >= 1 ? j - 1 + RB : RB - 1, NS - 1);
        wait_slices<RPL, RB - 2>(last - (j + 1));
      }
      wg_barrier();
    }
  } else {
    // ---- compute waves
    const int slot_i = __builtin_amdgcn_readfirstlane(wave / KP);  // wave-uniform
    const int kp = __builtin_amdgcn_readfirstlane(wave - slot_i * KP);
    const int r = lane & 15, kg = lane >> 4;
    const int tile = blockIdx.x + slot_i * gridDim.x;
    const bool active = tile < nT;
    const int t = active ? tile : nT - 1;
    const ST* __restrict__ sbp = reinterpret_cast<const ST*>(a.sb);
    const uint32_t* cbase = a.codes + ((long)t * nC) * 64 * BITS + lane * BITS;
    const ST* sbase = sbp + ((long)t * nC * kTileN + r) * 4;
    uint32_t W[DR][BITS];
    SBPair<ST> SBv[DR];
    auto load = [&](int s, int d) {
      const int c = min(s * KP + kp, nC - 1);
      const uint32_t* p = cbase + (long)c * 64 * BITS;
#pragma unroll
      for (int q = 0; q < BITS; ++q) W[d][q] = __builtin_nontemporal_load(p + q);
      SBv[d].load(sbase + (long)c * kTileN * 4);
    };
#pragma unroll
    for (int d = 0; d < DR; ++d)
      if (d < NS) load(d, d);
    const PairMasks mask_v = pair_mask_vgpr<BITS>();
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = zero;
    wg_barrier();
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int d = j % DR;
      const bool live = j * KP + kp < nC;
      const u32x4* slot = xs + (j % RB) * SLOT;
      uint32_t P[16];
      unpack_pairs<BITS>(W[d], P, mask_v);
      float sc[2], bp[2];
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        // group_affine() spelled out: this form keeps the kernel within 128 VGPRs
        const float s0 = SBv[d].s(gp);
        constexpr bool c3 = BITS == 3;
        sc[gp] = live ? (c3 && gp == 1 ? s0 * 0.125f : s0) : 0.f;
        bp[gp] = live ? SBv[d].b(gp) - (c3 && gp == 1 ? 16.f : 128.f) * s0 : 0.f;
      }
      // every activation read of the slice is issued before its first MFMA
      constexpr int MA = MT <= 2 ? MT : 2;  // m-tiles whose fragments are read together
#pragma unroll
      for (int m0 = 0; m0 < MT; m0 += MA) {
        u32x4 A[MA][4];
#pragma unroll
        for (int mi = 0; mi < MA; ++mi) {
          const u32x4* xrow = slot + (16 * (m0 + mi) + r) * 64;
#pragma unroll
          for (int q = 0; q < 4; ++q)  // vector of (chunk kp, group q>>1, quarter kg, half q&1)
            A[mi][q] = xrow[(16 * kp + 8 * (q >> 1) + 2 * kg + (q & 1)) ^ r];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mi = 0; mi < MA; ++mi) {
          const int mt = m0 + mi;
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            const f32x4 e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, A[mi][2 * gp]), __builtin_bit_cast(bf16x8, ones), zero, 0,
                0, 0);
            const f32x4 ex = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, A[mi][2 * gp + 1]), __builtin_bit_cast(bf16x8, ones), e, 0,
                0, 0);
            const u32x4 B0 = {P[8 * gp + 0], P[8 * gp + 1], P[8 * gp + 2], P[8 * gp + 3]};
            const u32x4 B1 = {P[8 * gp + 4], P[8 * gp + 5], P[8 * gp + 6], P[8 * gp + 7]};
            f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, A[mi][2 * gp]), __builtin_bit_cast(bf16x8, B0), zero, 0, 0,
                0);
            dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[mi][2 * gp + 1]),
                                                         __builtin_bit_cast(bf16x8, B1), dd, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[mt][q] = fmaf(sc[gp], dd[q], fmaf(bp[gp], ex[q], acc[mt][q]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j + DR < NS) load(j + DR, d);
      wait_lds();
      wg_barrier();
    }
    // fold the KP partial tiles of this tile slot in K order (slots are dead)
    f32x4* red = reinterpret_cast<f32x4*>(lds);  // [TM][MT][KP][64]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[((slot_i * MT + mt) * KP + kp) * 64 + lane] = acc[mt];
    __syncthreads();
    if (kp != 0 || !active) return;
    const int n = tile * kTileN + r;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 v = acc[mt];
#pragma unroll
      for (int i = 1; i < KP; ++i) v += red[((slot_i * MT + mt) * KP + i) * 64 + lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * mt + 4 * kg + q;
        if (m < M) store_y<false>(a, (long)m * a.ldy + n, v[q]);
      }
    }
    return;
  }
  __syncthreads();  // loader waves: partner of the compute waves' fold barrier
}

// ---------------------------------------------------------------------------
// Split slab kernel for 17..64 activation rows.  The slab kernel's loader /
// compute structure, changed where a 64-row block spends its time: every
// compute unit of the slab kernel takes in the whole activation block
// (655 KB at K = 5120) and reads each fragment from LDS once per W tile.
//   * K is cut into S parts (S = 1 or 2): workgroup (g, s) covers the
//     TG = NSLOT*TW W tiles of tile group g over the NS slices of part s, so
//     a compute unit takes in only its part of the activations;
//   * compute wave (slot, kp) serves TW tiles (chunk kp of every slice):
//     each A fragment it reads and each group sum (all-ones MFMA) it forms
//     serves TW tiles; a tile's packed weights are unpacked once per slice,
//     DR slices of weight loads are kept in flight in a register ring.
// The KP = 4 partial tiles of a tile are added through LDS in K order.  With
// S = 2 each workgroup then stores its partial tiles with device-coherent
// stores (written through to the point of coherence for the whole device,
// so no L2 write-back is needed), waits for them, and takes a ticket; the
// workgroup that arrives second adds the two partials (a + b is the same in
// either order) and writes y, then re-arms the ticket.  Workgroups are
// numbered g*S + s and dealt to the XCDs round-robin, so with S = 2 each
// XCD's L2 holds one part of the activation block.
// ---------------------------------------------------------------------------
template <int BITS, int MT, int TW, int NSLOT, int NS, int RB, int DR, typename ST>
__global__ void __launch_bounds__((NSLOT * 4 + 4) * 64) split_slab_kernel(LaunchArgs a) {
  constexpr int KP = 4, NWC = NSLOT * KP, NWL = 4;
  constexpr int ROWS = 16 * MT;
  constexpr int SK = KP * kChunkK;  // k per slice
  constexpr int SLOT = ROWS * 64;   // vectors per slot
  constexpr int RPL = ROWS / NWL;   // rows per loader wave per slice
  constexpr int NB = RB < NS ? RB : NS;
  constexpr int TG = NSLOT * TW;    // W tiles per workgroup
  static_assert(MT >= 2 && MT <= KP, "one folded row tile per compute wave");
  static_assert(TG * MT * KP * 1024 <= RB * SLOT * 16, "fold area exceeds the ring");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ int s_last;
  u32x4* xs = reinterpret_cast<u32x4*>(lds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nT = a.N / kTileN, nC = a.K / kChunkK;
  const int M = a.M, S = a.S;
  const int grp = blockIdx.x / S, kpart = blockIdx.x - grp * S;
  const int sl0 = kpart * NS;  // first slice of this workgroup's part of K
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const int slot_i = __builtin_amdgcn_readfirstlane(wave / KP);  // wave-uniform
  const int kp = __builtin_amdgcn_readfirstlane(wave - slot_i * KP);
  const int r = lane & 15, kg = lane >> 4;
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // fold area [TG][MT][KP][64], after the loop
  // timing build only: stamps after the partial tiles' words
  WaveStamps ts(a, (long)blockIdx.x * (NWC + NWL) + wave, (long)gridDim.x * TG * MT * 128);
  ts.mark(0);

  if (wave >= NWC) {
    // ---- loader waves
    const int lw = __builtin_amdgcn_readfirstlane(wave - NWC);  // wave-uniform
    const uint16_t* __restrict__ xg = reinterpret_cast<const uint16_t*>(a.x);
    auto issue = [&](int s) {
      u32x4* slot = xs + (s % RB) * SLOT;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const int m = lw + i * NWL;
        const int v = lane ^ (m & 15);
        const int col = min((sl0 + s) * SK + 8 * v, a.K - 8);
        const uint16_t* src = xg + (long)min(m, M - 1) * a.ldx + col;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)src,
            (__attribute__((address_space(3))) void*)(slot + m * 64), 16, 0, 0);
      }
    };
#pragma unroll
    for (int s = 0; s < NB; ++s) issue(s);
    wait_vm<(NB - 1) * RPL>();
    wg_barrier();
    ts.mark(1);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      // after barrier j every compute wave is done with slice j-1
      if (j >= 1 && j - 1 + RB < NS) issue(j - 1 + RB);
      if (j + 1 < NS) {
        const int last = min(j >= 1 ? j - 1 + RB : RB - 1, NS - 1);
        wait_slices<RPL, RB - 2>(last - (j + 1));
      }
      wg_barrier();
      ts.mark(2 + j);
    }
  } else {
    // ---- compute waves
    const ST* __restrict__ sbp = reinterpret_cast<const ST*>(a.sb);
    int tl[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) tl[i] = min(grp * TG + slot_i * TW + i, nT - 1);
    // weight ring: slice j's codes and scales/biases in slot j % DR
    uint32_t W[DR][TW][BITS];
    SBPair<ST> SBv[DR][TW];
    auto load = [&](int j) {
      const int c = min((sl0 + j) * KP + kp, nC - 1);
      const int d = j % DR;
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const uint32_t* p = a.codes + ((long)tl[i] * nC + c) * 64 * BITS + lane * BITS;
#pragma unroll
        for (int q = 0; q < BITS; ++q) W[d][i][q] = __builtin_nontemporal_load(p + q);
        SBv[d][i].load(sbp + ((long)tl[i] * nC * kTileN + r) * 4 + (long)c * kTileN * 4);
      }
    };
#pragma unroll
    for (int j = 0; j < DR; ++j)
      if (j < NS) load(j);
    const PairMasks mask_v = pair_mask_vgpr<BITS>();
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    f32x4 acc[TW][MT];
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[i][mt] = zero;
    wg_barrier();
    ts.mark(1);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const bool live = (sl0 + j) * KP + kp < nC;
      const u32x4* slot = xs + (j % RB) * SLOT;
      // group by group: only one group's unpacked pairs are live at a time
      // (the other half of each unpack is dead code); slice j + DR's weight
      // loads go out once the second group is unpacked
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        uint32_t P[TW][16];
        float sc[TW], bp[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          unpack_pairs<BITS>(W[j % DR][i], P[i], mask_v);
          const float s0 = SBv[j % DR][i].s(gp);
          constexpr bool c3 = BITS == 3;
          sc[i] = live ? (c3 && gp == 1 ? s0 * 0.125f : s0) : 0.f;
          bp[i] = live ? SBv[j % DR][i].b(gp) - (c3 && gp == 1 ? 16.f : 128.f) * s0 : 0.f;
        }
        if (gp == 1 && j + DR < NS) load(j + DR);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const u32x4* xrow = slot + (16 * mt + r) * 64;
          u32x4 A[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)  // vector of (chunk kp, group gp, quarter kg, half h)
            A[h] = xrow[(16 * kp + 8 * gp + 2 * kg + h) ^ r];
          __builtin_amdgcn_sched_barrier(0);
          const f32x4 e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, A[0]), __builtin_bit_cast(bf16x8, ones), zero, 0, 0, 0);
          const f32x4 ex = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, A[1]), __builtin_bit_cast(bf16x8, ones), e, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < TW; ++i) {
            const u32x4 B0 = {P[i][8 * gp + 0], P[i][8 * gp + 1], P[i][8 * gp + 2], P[i][8 * gp + 3]};
            const u32x4 B1 = {P[i][8 * gp + 4], P[i][8 * gp + 5], P[i][8 * gp + 6], P[i][8 * gp + 7]};
            f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, A[0]), __builtin_bit_cast(bf16x8, B0), zero, 0, 0, 0);
            dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[1]),
                                                         __builtin_bit_cast(bf16x8, B1), dd, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][mt][q] = fmaf(sc[i], dd[q], fmaf(bp[i], ex[q], acc[i][mt][q]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_lds();
      wg_barrier();
      ts.mark(2 + j);
    }
    // the slots are dead: park the partial tiles for the fold
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        red[(((slot_i * TW + i) * MT + mt) * KP + kp) * 64 + lane] = acc[i][mt];
  }
  __syncthreads();
  ts.mark(10);
  // wave (slot, kp) folds row tile mt = kp of its TW tiles in K order
  const bool folds = wave < NWC && kp < MT;
  const int mt = kp;
  f32x4 v[TW];
  if (folds) {
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const int base = ((slot_i * TW + i) * MT + mt) * KP;
      v[i] = red[base * 64 + lane];
#pragma unroll
      for (int k = 1; k < KP; ++k) v[i] += red[(base + k) * 64 + lane];
    }
  }
  ts.mark(11);
  auto store_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const int tile = grp * TG + slot_i * TW + i;
      if (tile >= nT) continue;
      const int n = tile * kTileN + r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * mt + 4 * kg + q;
        if (m < M) store_y<false>(a, (long)m * a.ldy + n, v[i][q]);
      }
    }
  };
  if (S == 1) {
    if (folds) store_tiles();
    ts.flush(lane);
    return;
  }
  // S == 2: partial tile (grp, kpart, slot, i, mt) at part[(((grp*S + kpart)*TG + slot*TW + i)*MT
  // + mt)*256 + q*64 + lane]
  auto part_at = [&](int kq, int i, int q) {
    return a.part + ((((long)(grp * S + kq) * TG + slot_i * TW + i) * MT + mt) * 4 + q) * 64 + lane;
  };
  if (folds) {
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __hip_atomic_store(part_at(kpart, i, q), v[i][q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vm<0>();  // the partials have reached the point of coherence
  }
  ts.mark(12);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&a.tickets[grp], 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(S - 1);
  __syncthreads();
  ts.mark(13);
  if (!s_last) {
    ts.flush(lane);
    return;
  }
  if (folds) {
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[i][q] += __hip_atomic_load(part_at(1 - kpart, i, q), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    store_tiles();
  }
  ts.mark(14);
  ts.flush(lane);
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.tickets[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// (row tiles, slices of 512 k) shapes of the slab kernel; three tile slots.
#define QMM_SLAB_SHAPES(X) X(1, 10) X(1, 16) X(2, 10) X(2, 16) X(4, 10) X(4, 16)

int slab_slices(int mt, int nC) {
  const int ns = (nC + 3) / 4;
#define QMM_HAS(MTV, NSV) if (mt == MTV && ns == NSV) return ns;
  QMM_SLAB_SHAPES(QMM_HAS)
#undef QMM_HAS
  return 0;
}

// LDS ring slots and weight ring depth (slices of loads in flight per
// compute wave), measured on the 3-bit 5120x10240 workload: deeper weight
// rings queue the activation slices behind weight loads and run slower.
// LDS ring slots per row-tile count (128 KB at one, two and four row tiles,
// 144 KB at three; three row tiles run in the split form only)
static constexpr int slab_ring(int mt) { return mt == 4 ? 2 : (mt == 3 ? 3 : 4); }
static constexpr int slab_depth(int mt) { return mt == 2 ? 2 : 3; }
size_t slab_lds_bytes(int mt) { return (size_t)slab_ring(mt) * 16 * mt * 1024; }

template <int BITS, typename ST>
static hipError_t slab_dispatch(int mt, int ns, const LaunchArgs& a, int grid, size_t lds,
                                hipStream_t st) {
#define QMM_SLAB(MTV, NSV)                                                                    \
  if (mt == MTV && ns == NSV) {                                                               \
    auto* kfn = &slab_kernel<BITS, MTV, kSlabTiles, NSV, slab_ring(MTV), slab_depth(MTV), ST>; \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                    \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    if (e != hipSuccess) return e;                                                            \
    kfn<<<grid, (kSlabTiles * 4 + 4) * 64, lds, st>>>(a);                                     \
    return hipGetLastError();                                                                 \
  }
  QMM_SLAB_SHAPES(QMM_SLAB)
#undef QMM_SLAB
  return hipErrorInvalidValue;
}

hipError_t launch_slab(int bits, bool sb_f32, int mt, int ns, const LaunchArgs& a, int grid,
                       size_t lds_bytes, hipStream_t st) {
  if (bits == 3)
    return sb_f32 ? slab_dispatch<3, float>(mt, ns, a, grid, lds_bytes, st)
                  : slab_dispatch<3, uint16_t>(mt, ns, a, grid, lds_bytes, st);
  return sb_f32 ? slab_dispatch<4, float>(mt, ns, a, grid, lds_bytes, st)
                : slab_dispatch<4, uint16_t>(mt, ns, a, grid, lds_bytes, st);
}

// (row tiles, slices per workgroup) and (tiles per wave, tile slots) shapes
// of the split slab kernel that are built: two K parts of K = 5120 or 8192
// (5 or 8 slices each), two W tiles per wave in three slots (three tiles per
// wave in two slots spills registers at four row tiles and measured no
// faster; one K part leaves half the compute units idle).
#define QMM_SPLIT_SLAB_SHAPES(X) X(2, 5) X(3, 5) X(4, 5) X(2, 8) X(3, 8) X(4, 8)
#define QMM_SPLIT_SLAB_WAVES(X) X(2, 3)

bool split_slab_shape(int mt, int tw, int nC, int S, int* ns, int* nslot) {
  if (S != 2 || nC % (4 * S) != 0) return false;
  const int want = nC / (4 * S);
  bool shape = false, waves = false;
#define QMM_HAS(MTV, NSV) if (mt == MTV && want == NSV) shape = true;
  QMM_SPLIT_SLAB_SHAPES(QMM_HAS)
#undef QMM_HAS
#define QMM_HASW(TWV, NSL) if (tw == TWV) { waves = true; *nslot = NSL; }
  QMM_SPLIT_SLAB_WAVES(QMM_HASW)
#undef QMM_HASW
  *ns = want;
  return shape && waves;
}

// weight ring depth: two slices ahead where the registers allow it
static constexpr int split_slab_depth(int mt) { return mt == 2 ? 2 : 1; }
size_t split_slab_lds_bytes(int mt) { return (size_t)slab_ring(mt) * 16 * mt * 1024; }

size_t split_slab_part_bytes(int mt, int tw, int nslot, int groups, int S) {
  return S > 1 ? (size_t)groups * S * tw * nslot * mt * 1024 : 0;
}

template <int BITS, typename ST>
static hipError_t split_slab_dispatch(int mt, int ns, int tw, const LaunchArgs& a, int grid,
                                      size_t lds, hipStream_t st) {
#define QMM_SSLAB_W(MTV, NSV, TWV, NSL)                                                      \
  if (mt == MTV && ns == NSV && tw == TWV) {                                                \
    auto* kfn = &split_slab_kernel<BITS, MTV, TWV, NSL, NSV, slab_ring(MTV),               \
                                   split_slab_depth(MTV), ST>;                             \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),                  \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    if (e != hipSuccess) return e;                                                          \
    kfn<<<grid, (NSL * 4 + 4) * 64, lds, st>>>(a);                                          \
    return hipGetLastError();                                                               \
  }
#define QMM_SSLAB(MTV, NSV) QMM_SSLAB_W(MTV, NSV, 2, 3)
  QMM_SPLIT_SLAB_SHAPES(QMM_SSLAB)
#undef QMM_SSLAB
#undef QMM_SSLAB_W
  return hipErrorInvalidValue;
}

hipError_t launch_split_slab(int bits, bool sb_f32, int mt, int ns, int tw, const LaunchArgs& a,
                             int grid, size_t lds_bytes, hipStream_t st) {
  if (bits == 3)
    return sb_f32 ? split_slab_dispatch<3, float>(mt, ns, tw, a, grid, lds_bytes, st)
                  : split_slab_dispatch<3, uint16_t>(mt, ns, tw, a, grid, lds_bytes, st);
  return sb_f32 ? split_slab_dispatch<4, float>(mt, ns, tw, a, grid, lds_bytes, st)
                : split_slab_dispatch<4, uint16_t>(mt, ns, tw, a, grid, lds_bytes, st);
}

}  // namespace qmm
