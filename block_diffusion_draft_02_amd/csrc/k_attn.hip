// Non-causal paged GQA block attention (memra_engine/dflash.rs, DflashDraft::forward_round:
// every block query sees every context key and every block key; scale 1/sqrt(head_dim);
// sliding layers additionally hide keys with q_pos - k_pos >= window).
//
// Work split: the keys of a band are cut into chunks whose length depends only on the band's
// own length (a multiple of 256 keys) and the drafter's create-time path switch, so a band's
// result does not depend on which other bands share the call. Two paths share one launch
// per layer, each band taking one by its own length (the LDS path, further below, streams a
// long band's K/V through LDS for all its query rows at once; a call whose bands all take it
// runs that path's own launch). The register path: one
// workgroup per (chunk, kv head, 32 query rows), with the band table passed by value. The
// workgroup stages its query rows (hi, lo) and all the chunk's page ids in LDS; each of its
// four wavefronts then takes 32-key slices of the chunk (keys 32w, 32w + 128, ...), loading a
// slice's K and V^T fragments straight from the pool into MFMA operands, and keeps an online
// softmax state (exp2 domain, running maximum in raw score units, so a probability is one FMA
// and one v_exp_f32) for its two 16-row query tiles:
//   S^T = K Q^T   two 16x16x32 MFMA tiles per slice and query tile; the key order inside
//                 the tiles is permuted so that every lane ends up holding 8 consecutive
//                 keys of one row
//   O^T += V^T P^T one MFMA per 16 head dims; P^T comes straight from the lane's own
//                 registers and V^T is one 16-byte load because V pages are stored [d][16]
// The four states are merged in wave order through LDS into one (max, sum, unnormalised O)
// partial per row and chunk; k_attn_combine merges the chunks of a band.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dfl {

constexpr int KW = 32;           // keys of one wavefront's slice per pass
constexpr int AW = 4;            // wavefronts per workgroup
constexpr int KP = AW * KW;      // keys of one workgroup pass
constexpr int RG = 32;           // query rows per workgroup: two 16-row tiles
constexpr int RPAD = ATTN_PART_ROWS;   // query-row slots of one (chunk, kv head) partial
constexpr int NCH_MAX = 64;      // chunks of one band that k_attn_combine accepts
constexpr float RESCALE_LOG2 = 8.f;  // headroom of the lazily moved softmax reference maximum
// ATTN_CHUNK_PAGES_MAX (kernels.hpp): page ids of a chunk, all staged in LDS

// LDS: the workgroup's query rows (hi, lo) during the key loop, then the four waves'
// partial states for the merge; plus the chunk's page ids
template <int HD>
struct AttnLds {
  union {
    struct {
      bf16 h[RG][HD + 8];   // rows padded by 16 B: 8 lanes reading 8 rows hit distinct banks
      bf16 l[RG][HD + 8];
    } q;
    struct {
      float o[AW][RG][HD + 4];
      float m[AW][RG];
      float l[AW][RG];
    } mg;
  };
  int page[ATTN_CHUNK_PAGES_MAX];
};

// one wave's 32-key slice in registers: K fragments of the two S^T tiles, V^T fragments,
// and (sliding layers) the stamped positions of the lane's 8 keys
template <int HD, bool WIN>
struct Slice {
  bf16x8 kf[2][HD / 32];
  bf16x8 vf[HD / 16];
  int kp[WIN ? 8 : 1];
};

template <int HD, bool WIN>
__device__ __forceinline__ void load_slice(Slice<HD, WIN>& sl, const AttnLds<HD>& sm,
                                           const bf16* __restrict__ lpool, const int* __restrict__ kpos,
                                           size_t pl, int kvh, int nkv, int npg, int kt, int c, int grp) {
  constexpr int NS = HD / 32, ND = HD / 16;
  // the slice's 32 keys lie on chunk pages kt/16 and kt/16 + 1 (the zeroed sentinel page 0
  // past the chunk, so every operand is finite and masked keys add exactly zero); the page
  // ids come from LDS only, so no load of the key loop waits on another
  const int lp = kt >> 4;
  const int p0 = sm.page[min(lp, ATTN_CHUNK_PAGES_MAX - 1)];
  const int p1 = lp + 1 < npg ? sm.page[min(lp + 1, ATTN_CHUNK_PAGES_MAX - 1)] : 0;
  // K fragments: S^T tile t, row c covers slice key (c/4)*8 + t*4 + c%4, so lane (c, grp)
  // of the result holds slice keys grp*8 + 0..7 of query row c (e = t*4 + slot)
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kk = (c >> 2) * 8 + t * 4 + (c & 3);
    const bf16* kp = lpool + (size_t)(kk >> 4 ? p1 : p0) * pl + ((size_t)kvh * PAGE + (kk & 15)) * HD + grp * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) sl.kf[t][s] = ld8(kp + s * 32);
  }
  // V^T fragments: row d = dt*16 + c, slice keys grp*8 + 0..7 (one 16-byte run of a [d][16]
  // V page)
  const int pv = grp >> 1 ? p1 : p0;
  const bf16* vp = lpool + (size_t)pv * pl + (size_t)(nkv + kvh) * HD * PAGE + c * PAGE + (grp & 1) * 8;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) sl.vf[dt] = ld8(vp + dt * 16 * PAGE);
  if (WIN) {
    const int* pp = kpos + (size_t)pv * PAGE + (grp & 1) * 8;
    const i32x4 a = *reinterpret_cast<const i32x4*>(pp), b = *reinterpret_cast<const i32x4*>(pp + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { sl.kp[e] = a[e]; sl.kp[(4 + e) & (WIN ? 7 : 0)] = b[e]; }
  }
}

template <int HD, bool WIN>
__device__ __forceinline__ void compute_slice(const Slice<HD, WIN>& sl, const AttnLds<HD>& sm, bool full, int lim,
                                              const int (&qpos)[2], int window, float scale_log2,
                                              float (&m_run)[2], float (&l_run)[2], f32x4 (&o)[2][HD / 16],
                                              int c, int grp) {
  constexpr int NS = HD / 32, ND = HD / 16;
  // S^T = K Q^T: four independent accumulator chains (query tile x key tile), each taking
  // the hi then the lo query term at every k-step
  f32x4 sh[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int t = 0; t < 2; ++t) sh[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const bf16x8 qh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.q.h[rt * 16 + c][s * 32 + grp * 8]));
#pragma unroll
      for (int t = 0; t < 2; ++t) sh[rt][t] = mfma16(sl.kf[t][s], qh, sh[rt][t]);
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const bf16x8 ql = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.q.l[rt * 16 + c][s * 32 + grp * 8]));
#pragma unroll
      for (int t = 0; t < 2; ++t) sh[rt][t] = mfma16(sl.kf[t][s], ql, sh[rt][t]);
    }
  }
  // online softmax in the exp2 domain with the running maximum kept in raw score units, so
  // each probability is one FMA and one v_exp_f32: p = 2^(s * scale - m * scale). Masks are
  // applied only where a key can be hidden (the chunk's last slice, sliding layers).
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = sh[rt][e >> 2][e & 3];
      if (WIN || !full) {
        bool ok = e < lim;
        if (WIN) ok = ok & (qpos[rt] - sl.kp[e & (WIN ? 7 : 0)] < window);
        x = ok ? x : -INFINITY;
      }
      sv[e] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // m_run is the row's reference maximum, not always the exact one: it moves (and the
    // running sum and output are rescaled) only when a score would exceed it by more than
    // 2^RESCALE_LOG2, so probabilities stay below 2^8 (exact in the fp32 sums and in bf16
    // range) and after the first slices the 64-register rescale almost never runs
    const bool move = tmax > m_run[rt] && (m_run[rt] == -INFINITY || (tmax - m_run[rt]) * scale_log2 > RESCALE_LOG2);
    if (__any(move)) {
      const float m_new = move ? tmax : m_run[rt];
      const float alpha = (m_new == -INFINITY || m_run[rt] == m_new) ? 1.f
                                                                     : __builtin_amdgcn_exp2f((m_run[rt] - m_new) * scale_log2);
      l_run[rt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) o[rt][dt] *= alpha;
      m_run[rt] = m_new;
    }
    // a row with every key so far hidden keeps m = -inf: its hidden scores still give 2^-inf = 0
    const float bias = (m_run[rt] == -INFINITY) ? 0.f : -m_run[rt] * scale_log2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], scale_log2, bias));
      l_run[rt] += sv[e];
    }
    // O^T += V^T P^T: P^T comes straight from the lane's own registers (bf16, round to nearest
    // even, two per instruction)
    const bf16x8 pb = __builtin_convertvector((f32x8){sv[0], sv[1], sv[2], sv[3], sv[4], sv[5], sv[6], sv[7]}, bf16x8);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[rt][dt] = mfma16(sl.vf[dt], pb, o[rt][dt]);
  }
}


// the band of a path's chunk cd: the band of that path whose chunks cover cd
__device__ __forceinline__ int attn_band(const AttnBands& ab, int cd, bool lds, int sw) {
  int bl = 0;
  for (int b = 0; b < ab.n; ++b)
    if ((((ab.lds_mask >> b) & 1u) != 0) == lds && cd >= ab.dbase[b] && cd < ab.dbase[b] + ab.b[b].nch[sw]) bl = b;
  return bl;
}

// the register path's workgroup `id` (ids counted from the first register-path workgroup)
template <int HD, bool WIN>
__device__ __forceinline__ void attn_reg_wg(AttnLds<HD>& sm, int id, const bf16* __restrict__ Q,
                                            const bf16* __restrict__ Q_lo, const AttnBands& ab, int n_items,
                                            int nrg, int gamma, int nh, const KvGeom& g, int layer, int sw,
                                            int window, float scale_log2, float* __restrict__ part_o,
                                            float* __restrict__ part_ml) {
  constexpr int ND = HD / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, grp = lane >> 4;
  // Workgroups are handed to the eight XCDs round robin, so ids 8 apart share an XCD and its
  // L2: the row groups of one (chunk, kv head) item get ids 8 apart and read its K/V from
  // HBM once.
  const int qd = id >> 3;
  const int rg = qd % nrg;
  const int item = (qd / nrg) * 8 + (id & 7);
  if (item >= n_items) return;
  const int nkv = g.nkv;
  const int cd = item / nkv, kvh = item - cd * nkv;
  const int G = nh / nkv;
  const int bl = attn_band(ab, cd, false, sw), b = bl;
  const int seq = ab.b[bl].seq, C = ab.b[bl].kv_len, qpos0 = ab.b[bl].q_pos;
  const int ch = cd - ab.dbase[bl];
  const size_t pitem = (size_t)(ab.b[bl].base[sw] + ch) * nkv + kvh;   // the call-wide partial slot
  const int k0 = ab.b[bl].kstart[sw] + ch * ab.b[bl].ck[sw];   // page aligned
  const int k1 = min(k0 + ab.b[bl].ck[sw], C + gamma);
  const int nkeys = k1 - k0;
  const int npg = (nkeys + PAGE - 1) / PAGE;
  const int R = gamma * G;
  const size_t pl = page_layer_elems(nkv, HD);
  const bf16* lpool = g.pool + (size_t)layer * g.num_pages * pl;
  const int* bt = g.bt + (size_t)seq * g.per_seq + (k0 >> 4);

  // the chunk's page ids and this workgroup's query rows (row r = rg*32 + rr is block row
  // r % gamma of query head r / gamma of this kv head's group; rows past R are zero)
  for (int i = threadIdx.x; i < min(npg, ATTN_CHUNK_PAGES_MAX); i += AW * 64) sm.page[i] = bt[i];
  for (int pc = threadIdx.x; pc < RG * HD / 8; pc += AW * 64) {
    const int rr = pc / (HD / 8), d8 = (pc % (HD / 8)) * 8;
    const int r = rg * RG + rr;
    u32x4 vh = u32x4{0u, 0u, 0u, 0u}, vl = vh;
    if (r < R) {
      const size_t qo = ((size_t)(b * gamma + r % gamma) * nh + kvh * G + r / gamma) * HD + d8;
      vh = *reinterpret_cast<const u32x4*>(Q + qo);
      vl = *reinterpret_cast<const u32x4*>(Q_lo + qo);
    }
    *reinterpret_cast<u32x4*>(&sm.q.h[rr][d8]) = vh;
    *reinterpret_cast<u32x4*>(&sm.q.l[rr][d8]) = vl;
  }
  int qpos[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) qpos[rt] = qpos0 + ((rg * RG + rt * 16 + c) % gamma);
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  f32x4 o[2][ND];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  // this wave's slices: keys kt = 32w, 32w + 128, ... (two waves per SIMD, and a second
  // workgroup per CU, cover the load latency and overlap one wave's softmax with the other's
  // MFMAs; a register ring of further slices would need one wave per SIMD, which loses that
  // overlap and measured slower)
  for (int kt = wave * KW; kt < nkeys; kt += KP) {
    Slice<HD, WIN> sl;
    load_slice<HD, WIN>(sl, sm, lpool, g.kpos, pl, kvh, nkv, npg, kt, c, grp);
    compute_slice<HD, WIN>(sl, sm, nkeys - kt >= KW, nkeys - kt - grp * 8, qpos, window, scale_log2, m_run, l_run, o,
                           c, grp);
  }

  // merge the four waves' states in wave order (the LDS now holds the merge area)
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float lt = l_run[rt];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
      *reinterpret_cast<f32x4*>(&sm.mg.o[wave][rt * 16 + c][dt * 16 + 4 * grp]) = o[rt][dt];
    if (grp == 0) {
      sm.mg.m[wave][rt * 16 + c] = m_run[rt] * scale_log2;   // the merge works in the exp2 domain
      sm.mg.l[wave][rt * 16 + c] = lt;
    }
  }
  __syncthreads();
  constexpr int DS = HD / 8;   // dims per thread: 8 threads per row
  const int row = threadIdx.x >> 3, slc = threadIdx.x & 7;
  const int r = rg * RG + row;
  if (r >= R) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < AW; ++w) M = fmaxf(M, sm.mg.m[w][row]);
  float wt[AW], L = 0.f;
#pragma unroll
  for (int w = 0; w < AW; ++w) {
    const float mw = sm.mg.m[w][row];
    wt[w] = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    L += wt[w] * sm.mg.l[w][row];
  }
  float* po = part_o + (pitem * RPAD + r) * HD + slc * DS;
#pragma unroll
  for (int v = 0; v < DS / 4; ++v) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < AW; ++w) acc += wt[w] * *reinterpret_cast<const f32x4*>(&sm.mg.o[w][row][slc * DS + v * 4]);
    *reinterpret_cast<f32x4*>(po + v * 4) = acc;
  }
  if (slc == 0) {
    part_ml[(pitem * RPAD + r) * 2 + 0] = M;
    part_ml[(pitem * RPAD + r) * 2 + 1] = L;
  }
}

// ---- K/V staged through LDS (head_dim 128, layers without a window, bands past 2048 keys) --
// One workgroup per (chunk, kv head) with all of the item's query rows, in waves of RT 16-row
// tiles (Q hi and lo held in registers): in the launch shared with the register path 4 waves
// of two tiles, in the LDS path's own launch 8 waves of one. Every wave takes every 32-key
// slice of the chunk in order, so the chunk's K/V leaves L2 once instead of once per row
// group. Slices stream through a ring of LDS slots with the gfx950 global->LDS 16-byte load,
// which takes no registers: a slice's four 4 KB pages (K of keys 0-15 and 16-31, then V) are
// sixteen 1 KB instructions shared out over the waves, each lane choosing its source so that
// the LDS copy is swizzled for the MFMA fragment reads (K: 16-byte unit u of row r of page p
// sits at unit u ^ (r ^ 4p); V: half h of dim row d sits at half h ^ (d/8 % 2)). Slice j + 2
// is requested right after the barrier that ends slice j - 1, and a wave waits (vmcnt) only
// for its own loads of slice j: one barrier per slice. A wave's state covers its rows over the
// whole chunk, so it writes the chunk's partials itself. Chunks start longest first.
constexpr int DMA_HD = 128;
constexpr int DMA_RING = 3;   // ring slots (a fourth measured no faster in either launch)

struct DmaSlice {
  bf16 k[2][PAGE * DMA_HD];   // two K pages [16 keys][128], units swizzled within a row
  bf16 v[2][DMA_HD * PAGE];   // two V pages [128 dims][16 keys], halves swizzled
};

// s_waitcnt with vmcnt <= N (vmcnt[3:0] | vmcnt[5:4] << 14; expcnt and lgkmcnt left at maximum)
#define DFL_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))

// One slice for a wave's RT row tiles. `loadv` reads the slice's V fragments from LDS: with two
// tiles before the scores (both tiles' products use them), with one only after the softmax,
// when the K fragments are dead, so that a wave fits in 128 registers.
template <int RT, class LoadV>
__device__ __forceinline__ void compute_dma(const bf16x8 (&kf)[2][4], LoadV&& loadv, const bf16x8 (&qh)[RT][4],
                                            const bf16x8 (&ql)[RT][4], bool full, int lim, float scale_log2,
                                            float (&m_run)[RT], float (&l_run)[RT], f32x4 (&o)[RT][8]) {
  bf16x8 vf[8];
  if constexpr (RT > 1) loadv(vf);
  // S^T = K Q^T, the hi then the lo query term at every k-step (as the register kernel)
  f32x4 sh[RT][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < 2; ++t) sh[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < 2; ++t) sh[rt][t] = mfma16(kf[t][s], qh[rt][s], sh[rt][t]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < 2; ++t) sh[rt][t] = mfma16(kf[t][s], ql[rt][s], sh[rt][t]);
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = sh[rt][e >> 2][e & 3];
      if (!full) x = e < lim ? x : -INFINITY;
      sv[e] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const bool move = tmax > m_run[rt] && (m_run[rt] == -INFINITY || (tmax - m_run[rt]) * scale_log2 > RESCALE_LOG2);
    if (__any(move)) {
      const float m_new = move ? tmax : m_run[rt];
      const float alpha = (m_new == -INFINITY || m_run[rt] == m_new) ? 1.f
                                                                     : __builtin_amdgcn_exp2f((m_run[rt] - m_new) * scale_log2);
      l_run[rt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[rt][dt] *= alpha;
      m_run[rt] = m_new;
    }
    const float bias = (m_run[rt] == -INFINITY) ? 0.f : -m_run[rt] * scale_log2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], scale_log2, bias));
      l_run[rt] += sv[e];
    }
    const bf16x8 pb = __builtin_convertvector((f32x8){sv[0], sv[1], sv[2], sv[3], sv[4], sv[5], sv[6], sv[7]}, bf16x8);
    if constexpr (RT == 1) loadv(vf);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[rt][dt] = mfma16(vf[dt], pb, o[rt][dt]);
  }
}

template <int NR>
struct DmaLdsT {
  DmaSlice ring[NR];
  int page[ATTN_CHUNK_PAGES_MAX];
};
using DmaLds = DmaLdsT<DMA_RING>;

// wait until at most `ahead` slices' loads (IPW instructions each) of this wave are in flight
template <int IPW>
__device__ __forceinline__ void wait_slices(int ahead) {
  if (ahead >= 3) DFL_WAIT_VM(3 * IPW);
  else if (ahead == 2) DFL_WAIT_VM(2 * IPW);
  else if (ahead == 1) DFL_WAIT_VM(IPW);
  else DFL_WAIT_VM(0);
}

// the LDS path's workgroup `item` (one per (chunk, kv head) of the LDS-path bands): 8 / RT
// waves, each with RT 16-row tiles of the item's query rows, slices through a ring of NR slots
// (NR - 1 requested ahead)
template <int RT, int NR>
__device__ __forceinline__ void attn_lds_wg(DmaLdsT<NR>& sm, int item, const bf16* __restrict__ Q,
                                            const bf16* __restrict__ Q_lo, const AttnBands& ab, int gamma, int nh,
                                            const KvGeom& g, int layer, float scale_log2,
                                            float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int HD = DMA_HD, NS = HD / 32, ND = HD / 16, UPR = HD / 8;
  constexpr int NW = 8 / RT, IPW = 16 / NW;   // waves; 1 KB load instructions a wave and slice
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, grp = lane >> 4;
  const int nkv = g.nkv;
  const int cd = item / nkv, kvh = item - cd * nkv;
  const int G = nh / nkv;
  int run = 0;   // the dispatch run holding cd
  while (run + 1 < ab.n_lg && cd >= ab.lg_start[run + 1]) ++run;
  const int bl = ab.lg_band[run], b = bl;
  const int seq = ab.b[bl].seq, C = ab.b[bl].kv_len;
  const int ch = ab.lg_chunk[run] + (cd - ab.lg_start[run]);
  const size_t pitem = (size_t)(ab.b[bl].base[0] + ch) * nkv + kvh;   // the call-wide partial slot
  const int k0 = ab.b[bl].kstart[0] + ch * ab.b[bl].ck[0];   // page aligned
  const int k1 = min(k0 + ab.b[bl].ck[0], C + gamma);
  const int nkeys = k1 - k0;
  const int npg = (nkeys + PAGE - 1) / PAGE;
  const int R = gamma * G;
  const bool active = wave * 16 * RT < R;   // waves past the query rows only move K/V
  const size_t pl = page_layer_elems(nkv, HD);
  const bf16* lpool = g.pool + (size_t)layer * g.num_pages * pl;
  const int* bt = g.bt + (size_t)seq * g.per_seq + (k0 >> 4);
  // this wave's query rows r = 16 (RT wave + rt) + c (block row r % gamma of query head
  // r / gamma of the kv head's group; rows past R are zero) as S^T operands: dims
  // s*32 + grp*8 .. +7
  bf16x8 qh[RT][NS], ql[RT][NS];
  float m_run[RT], l_run[RT];
  f32x4 o[RT][ND];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) m_run[rt] = -INFINITY, l_run[rt] = 0.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the query rows first, so that their loads overlap the page ids'
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = (wave * RT + rt) * 16 + c;
    const size_t qo = ((size_t)(b * gamma + r % gamma) * nh + kvh * G + r / gamma) * HD + grp * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qh[rt][s] = r < R ? ld8(Q + qo + s * 32) : bf16x8{};
      ql[rt][s] = r < R ? ld8(Q_lo + qo + s * 32) : bf16x8{};
    }
  }
  for (int i = threadIdx.x; i < min(npg, ATTN_CHUNK_PAGES_MAX); i += NW * 64) sm.page[i] = bt[i];
  __syncthreads();   // the page ids
  DFL_WAIT_VM(0);    // and the query rows, in every wave, before the first slice is requested

  const int nsl = (nkeys + 31) / 32;
  // request slice j into ring slot d: the slice's four pages (K0, K1, V0, V1; the zeroed
  // sentinel page 0 past the chunk) are 16 1 KB instructions, IPW of them this wave's:
  // instruction q of page (wave IPW + i) / 4, q = (wave IPW + i) % 4
  auto issue = [&](DmaSlice& d, int j) {
    constexpr int PPW = IPW >= 4 ? IPW / 4 : 1;   // pages a wave touches
#pragma unroll
    for (int pi = 0; pi < PPW; ++pi) {
      const int pg = (wave * IPW) / 4 + pi;
      const int p = pg & 1;
      const int lp = j * 2 + p;
      const int pgid = lp < npg ? sm.page[min(lp, ATTN_CHUNK_PAGES_MAX - 1)] : 0;
      constexpr int QN = IPW >= 4 ? 4 : IPW;
      const int q0 = IPW >= 4 ? 0 : (wave * IPW) % 4;
      if (pg < 2) {
        const bf16* src = lpool + (size_t)pgid * pl + (size_t)kvh * PAGE * HD;
#pragma unroll
        for (int qi = 0; qi < QN; ++qi) {
          const int P = (q0 + qi) * 64 + lane;
          const int rr = P / UPR, u = (P % UPR) ^ ((rr ^ (4 * p)) & (UPR - 1));
          __builtin_amdgcn_global_load_lds(src + rr * HD + u * 8, &d.k[p][(q0 + qi) * 512], 16, 0, 0);
        }
      } else {
        const bf16* src = lpool + (size_t)pgid * pl + (size_t)(nkv + kvh) * HD * PAGE;
#pragma unroll
        for (int qi = 0; qi < QN; ++qi) {
          const int P = (q0 + qi) * 64 + lane;
          const int dd = P >> 1, h = (P & 1) ^ ((dd >> 3) & 1);
          __builtin_amdgcn_global_load_lds(src + dd * PAGE + h * 8, &d.v[p][(q0 + qi) * 512], 16, 0, 0);
        }
      }
    }
  };
  // one slice: this wave's loads of slice j are done once at most those of slices j + 1 ..
  // j + NR - 2 are in flight; the barrier then makes every wave's share visible and ends every
  // wave's reads of the slot (nxt, slice j - 1's) that slice j + NR - 1 now overwrites
  auto step = [&](int j, const DmaSlice& sl, DmaSlice& nxt) {
    wait_slices<IPW>(min(NR - 2, nsl - 1 - j));
    __builtin_amdgcn_s_barrier();
    if (j + NR - 1 < nsl) issue(nxt, j + NR - 1);
    if (!active) return;
    bf16x8 kf[2][NS];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kk = (c >> 2) * 8 + t * 4 + (c & 3);
      const int p = kk >> 4, rr = kk & 15;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int u = (4 * s + grp) ^ ((rr ^ (4 * p)) & (UPR - 1));
        kf[t][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sl.k[p][rr * HD + u * 8]));
      }
    }
    auto loadv = [&](bf16x8 (&vf)[ND]) {
      const int p = grp >> 1, h = grp & 1;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const int dd = dt * 16 + c;
        const int hq = h ^ ((dd >> 3) & 1);
        vf[dt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sl.v[p][dd * PAGE + hq * 8]));
      }
    };
    const int kt = j * 32;
    compute_dma<RT>(kf, loadv, qh, ql, nkeys - kt >= 32, nkeys - kt - grp * 8, scale_log2, m_run, l_run, o);
  };
  // slices 0 .. NR - 2 in flight before the loop (the query rows are already in registers, so
  // no load but the ring's is pending inside it)
#pragma unroll
  for (int i = 0; i < NR - 1; ++i)
    if (i < nsl) issue(sm.ring[i], i);
  for (int j0 = 0; j0 < nsl; j0 += NR) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (j0 + r < nsl) step(j0 + r, sm.ring[r], sm.ring[(r + NR - 1) % NR]);
  }

  // the wave's state is the chunk's partial of its rows (maximum in the exp2 domain)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = (wave * RT + rt) * 16 + c;
    float lt = l_run[rt];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (r >= R) continue;
    float* po = part_o + (pitem * RPAD + r) * HD + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[rt][dt];
    if (grp == 0) {
      part_ml[(pitem * RPAD + r) * 2 + 0] = m_run[rt] * scale_log2;
      part_ml[(pitem * RPAD + r) * 2 + 1] = lt;
    }
  }
}

// One launch per layer: the LDS-path workgroups first (their chunks are the long ones), then
// the register path's. The LDS holds either path's layout.
template <int HD, bool WIN>
struct AttnShm {
  AttnLds<HD> r;
};
template <>
struct AttnShm<DMA_HD, false> {
  union {
    AttnLds<DMA_HD> r;
    DmaLds d;
  };
};

template <int HD, bool WIN>
__global__ __launch_bounds__(AW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_block_attn(
    const bf16* __restrict__ Q, const bf16* __restrict__ Q_lo, const AttnBands ab, int n_lds_items, int n_items,
    int nrg, int gamma, int nh, KvGeom g, int layer, int sw, int window, float scale_log2,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) AttnShm<HD, WIN> sm;
  const int id = blockIdx.x;
  if constexpr (HD == DMA_HD && !WIN) {
    if (id < n_lds_items) {
      attn_lds_wg<2, DMA_RING>(sm.d, id, Q, Q_lo, ab, gamma, nh, g, layer, scale_log2, part_o, part_ml);
      return;
    }
  }
  attn_reg_wg<HD, WIN>(sm.r, id - n_lds_items, Q, Q_lo, ab, n_items, nrg, gamma, nh, g, layer, sw, window,
                       scale_log2, part_o, part_ml);
}


// The LDS path alone (a plan with no register-path chunk): eight waves of one 16-row tile
// each, held to 128 registers, so that with the ring and page ids alone in LDS (50 KB) two
// workgroups share a CU at four waves a SIMD.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_block_attn_lds(
    const bf16* __restrict__ Q, const bf16* __restrict__ Q_lo, const AttnBands ab, int gamma, int nh, KvGeom g,
    int layer, float scale_log2, float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) DmaLds sm;
  attn_lds_wg<1, DMA_RING>(sm, blockIdx.x, Q, Q_lo, ab, gamma, nh, g, layer, scale_log2, part_o, part_ml);
}

void plan_attn(const Band* bands, int n, int sw, int hd, int window, bool lds_path, int gamma, AttnBands& out,
               int& reg_chunks, int& lds_chunks) {
  const bool lds_ok = lds_path && hd == DMA_HD && window <= 0 && sw == 0;
  out.n = n;
  out.lds_mask = 0u;
  reg_chunks = lds_chunks = 0;
  int order[MAX_BANDS];
  for (int b = 0; b < n; ++b) {
    out.b[b] = bands[b];
    const int pages = (bands[b].kv_len + gamma - bands[b].kstart[sw] + PAGE - 1) / PAGE;
    if (lds_ok && pages > ATTN_LDS_MIN_PAGES) out.lds_mask |= 1u << b;
    order[b] = b;
  }
  // each path's chunks are numbered band by band, the bands with the longest chunks first, so
  // the longest workgroups start first (the dispatch order only; no band's sums change)
  // (a stable insertion sort: at most 32 bands, and no temporary buffer is allocated)
  for (int i = 1; i < n; ++i) {
    const int b = order[i];
    int j = i;
    for (; j > 0 && bands[order[j - 1]].ck[sw] < bands[b].ck[sw]; --j) order[j] = order[j - 1];
    order[j] = b;
  }
  for (int i = 0; i < n; ++i) {
    const int b = order[i];
    int& nch = (out.lds_mask >> b) & 1u ? lds_chunks : reg_chunks;
    out.dbase[b] = nch;
    nch += bands[b].nch[sw];
  }
  // the LDS path's dispatch order: every chunk longest first. A band's full chunks form one
  // run (in the order above, whose chunk widths fall), its last chunk another; the last chunks
  // are sorted by their own length and merged in (full runs first on ties). Only the order in
  // which workgroups start changes: a chunk's partial slot stays base + chunk.
  out.n_lg = 0;
  if (lds_chunks == 0) return;
  int last[MAX_BANDS], nl = 0;
  auto last_len = [&](int b) {
    const Band& B = bands[b];
    return B.kv_len + gamma - B.kstart[sw] - (B.nch[sw] - 1) * B.ck[sw];
  };
  for (int i = 0; i < n; ++i) {
    const int b = order[i];
    if (!((out.lds_mask >> b) & 1u)) continue;
    int j = nl++;
    for (; j > 0 && last_len(last[j - 1]) < last_len(b); --j) last[j] = last[j - 1];
    last[j] = b;
  }
  int pos = 0, il = 0;
  auto run = [&](int b, int c0, int cnt) {
    out.lg_start[out.n_lg] = (unsigned short)pos;
    out.lg_band[out.n_lg] = (unsigned char)b;
    out.lg_chunk[out.n_lg] = (unsigned char)c0;
    ++out.n_lg;
    pos += cnt;
  };
  for (int i = 0; i < n; ++i) {
    const int b = order[i];
    if (!((out.lds_mask >> b) & 1u) || bands[b].nch[sw] < 2) continue;
    while (il < nl && last_len(last[il]) > bands[b].ck[sw]) run(last[il], bands[last[il]].nch[sw] - 1, 1), ++il;
    run(b, 0, bands[b].nch[sw] - 1);
  }
  while (il < nl) run(last[il], bands[last[il]].nch[sw] - 1, 1), ++il;
  out.lg_start[out.n_lg] = (unsigned short)pos;
}

hipError_t launch_block_attn(const bf16* Q, const bf16* Q_lo, const AttnBands& bands, int reg_chunks, int lds_chunks,
                             int gamma, int nh, KvGeom g, int layer, int sw, int window,
                             float scale_log2, float* part_o, float* part_ml, hipStream_t st) {
  const int G = nh / g.nkv;
  const int R = gamma * G;
  if (R > RPAD || R < 1 || reg_chunks < 0 || lds_chunks < 0 || reg_chunks + lds_chunks < 1 || bands.n < 1 ||
      bands.n > MAX_BANDS)
    return hipErrorInvalidValue;
  if (lds_chunks > 0 && (g.hd != DMA_HD || window > 0 || sw != 0)) return hipErrorInvalidValue;
  const int n_items = reg_chunks * g.nkv, n_lds = lds_chunks * g.nkv;
  if (n_items == 0) {
    (void)launch(k_block_attn_lds, dim3(n_lds), 512, 0, st, Q, Q_lo, bands, gamma, nh, g, layer, scale_log2, part_o,
                 part_ml);
    return hipGetLastError();
  }
  const int nrg = (R + RG - 1) / RG;
  const dim3 grid(n_lds + ((n_items + 7) / 8) * 8 * nrg);
#define DFL_ATTN(HDV, W) (void)launch(k_block_attn<HDV, W>, grid, AW * 64, 0, st, Q, Q_lo, bands, n_lds, n_items, nrg, gamma, nh, g, layer, sw, window, scale_log2, part_o, part_ml)
  const bool win = window > 0;
  switch (g.hd) {
    case 128: if (win) DFL_ATTN(128, true); else DFL_ATTN(128, false); break;
    case 64: if (win) DFL_ATTN(64, true); else DFL_ATTN(64, false); break;
    case 32: if (win) DFL_ATTN(32, true); else DFL_ATTN(32, false); break;
    default: return hipErrorInvalidValue;
  }
#undef DFL_ATTN
  return hipGetLastError();
}

// Merge a band's chunk partials into the attention output (hi + lo bf16 terms). One
// workgroup per (band, kv head, RB blocks of CMB_ROWS query rows; blocks of four rows, so
// that even one band spreads over 128 workgroups); thread (row, 4-float slice, chunk group q)
// folds chunks q, q + CQ, q + 2CQ, ... (JM slots, at least the band's chunk count over CQ)
// with a running maximum, all of its loads issued at once; the CQ groups are then merged in
// group order. The order depends only on the band's own chunk count: JM and RB change how
// many loads a thread has in flight, not what any output element adds in which order.
constexpr int CMB_ROWS = 4;
template <int HD, int JM, int RB>
__global__ __launch_bounds__(1024) void k_attn_combine(const float* __restrict__ part_o,
                                                       const float* __restrict__ part_ml,
                                                       const Band* __restrict__ bands, int gamma,
                                                       int nh, int nkv, int sw,
                                                       bf16* __restrict__ out,
                                                       bf16* __restrict__ out_lo) {
  constexpr int NSL = HD / 4;             // 4-float slices per row
  constexpr int CR = CMB_ROWS;
  constexpr int CQ = 1024 / (CR * NSL);   // chunk groups
  __shared__ f32x4 red_o[RB][CQ][CR][NSL];
  __shared__ float red_m[RB][CQ][CR], red_l[RB][CQ][CR];
  const int b = blockIdx.x, kvh = blockIdx.y;
  const int q = threadIdx.x / (CR * NSL);
  const int row = (threadIdx.x / NSL) % CR, slc = threadIdx.x % NSL;
  const int G = nh / nkv;
  const int R = gamma * G;
  const int nch = bands[b].nch[sw], base = bands[b].base[sw];
  float mc[RB][JM], lc[RB][JM];
  f32x4 oc[RB][JM];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = (blockIdx.z * RB + rb) * CR + row;
#pragma unroll
    for (int j = 0; j < JM; ++j) {
      const int cc = q + j * CQ;
      if (r < R && cc < nch) {
        const size_t it = ((size_t)(base + cc) * nkv + kvh) * RPAD + r;
        mc[rb][j] = part_ml[it * 2];
        lc[rb][j] = part_ml[it * 2 + 1];
        oc[rb][j] = *reinterpret_cast<const f32x4*>(part_o + it * HD + slc * 4);
      } else {
        mc[rb][j] = -INFINITY;
        lc[rb][j] = 0.f;
        oc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < JM; ++j) M = fmaxf(M, mc[rb][j]);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
#pragma unroll
    for (int j = 0; j < JM; ++j) {
      const float w = (mc[rb][j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mc[rb][j] - M);
      acc += w * oc[rb][j];
      L += w * lc[rb][j];
    }
    red_o[rb][q][row][slc] = acc;
    if (slc == 0) {
      red_m[rb][q][row] = M;
      red_l[rb][q][row] = L;
    }
  }
  __syncthreads();
  if (q != 0) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = (blockIdx.z * RB + rb) * CR + row;
    if (r >= R) continue;
    float Mt = -INFINITY;
#pragma unroll
    for (int g2 = 0; g2 < CQ; ++g2) Mt = fmaxf(Mt, red_m[rb][g2][row]);
    f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
    float Lt = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < CQ; ++g2) {
      const float mg = red_m[rb][g2][row];
      const float w = (mg == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mg - Mt);
      tot += w * red_o[rb][g2][row][slc];
      Lt += w * red_l[rb][g2][row];
    }
    const float inv = 1.f / Lt;
    const int i = r % gamma, hq = r / gamma;
    const size_t o = ((size_t)(b * gamma + i) * nh + kvh * G + hq) * HD + slc * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) split_bf16(tot[e] * inv, out[o + e], out_lo[o + e]);
  }
}

template <int HD>
hipError_t launch_combine_hd(const float* part_o, const float* part_ml, const Band* bands_dev, int n_bands,
                             int max_nch, int gamma, int nh, int nkv, int sw, bf16* out, bf16* out_lo,
                             hipStream_t st) {
  constexpr int CQ = 1024 / (CMB_ROWS * (HD / 4));
  constexpr int JS = (16 + CQ - 1) / CQ;   // slots for bands of up to 16 chunks
  constexpr int JX = NCH_MAX / CQ;         // slots for any band
  const int groups = (gamma * (nh / nkv) + CMB_ROWS - 1) / CMB_ROWS;
  // four row blocks a workgroup once the call has rows for 2048 or more single blocks (then
  // every thread keeps 4 JS loads in flight and the launch fills the chip in about two rounds)
  const bool wide = max_nch <= JS * CQ && (long long)n_bands * nkv * groups >= 2048;
  if (wide) {
    const dim3 grid(n_bands, nkv, (groups + 3) / 4);
    (void)launch(k_attn_combine<HD, JS, 4>, grid, 1024, 0, st, part_o, part_ml, bands_dev, gamma, nh, nkv, sw, out, out_lo);
  } else if (max_nch <= JS * CQ) {
    (void)launch(k_attn_combine<HD, JS, 1>, dim3(n_bands, nkv, groups), 1024, 0, st, part_o, part_ml, bands_dev,
                 gamma, nh, nkv, sw, out, out_lo);
  } else {
    (void)launch(k_attn_combine<HD, JX, 1>, dim3(n_bands, nkv, groups), 1024, 0, st, part_o, part_ml, bands_dev,
                 gamma, nh, nkv, sw, out, out_lo);
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const float* part_o, const float* part_ml, const Band* bands_dev,
                               int n_bands, int max_nch, int gamma, int nh, int nkv, int hd, int sw,
                               bf16* out, bf16* out_lo, hipStream_t st) {
  if (max_nch < 1 || max_nch > NCH_MAX) return hipErrorInvalidValue;
  switch (hd) {
    case 32: return launch_combine_hd<32>(part_o, part_ml, bands_dev, n_bands, max_nch, gamma, nh, nkv, sw, out, out_lo, st);
    case 64: return launch_combine_hd<64>(part_o, part_ml, bands_dev, n_bands, max_nch, gamma, nh, nkv, sw, out, out_lo, st);
    case 128: return launch_combine_hd<128>(part_o, part_ml, bands_dev, n_bands, max_nch, gamma, nh, nkv, sw, out, out_lo, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dfl
