// Non-causal paged GQA block attention (memra_engine/dflash.rs, DflashDraft::forward_round:
// every block query sees every context key and every block key; scale 1/sqrt(head_dim);
// sliding layers additionally hide keys with q_pos - k_pos >= window).
//
// Work split: one workgroup per (band, kv head, key chunk of at most 256 keys). The chunk
// streams through two 64-key LDS buffers: the next step's K rows and V pages are in flight
// while the current step is computed. The four wavefronts own the band's gamma * G query
// rows of that kv head (G = query heads per kv head), two 16-row tiles each, so every K and
// V fragment read from LDS feeds two MFMAs. Per 64-key step and row tile:
//   S^T = K Q^T   four 16x16x32 MFMA tiles; the key order inside the tiles is permuted so
//                 that every lane ends up holding 8 consecutive keys of one row
//   online softmax per row (exp2 domain), lane-local partial sums
//   O^T += V^T P^T one MFMA per 16 head dims; P^T comes straight from the lane's own
//                 registers and V^T is one 16-byte load because V pages are stored [d][16]
// Each chunk leaves (max, sum, unnormalised O) per row; k_attn_combine merges the chunks of
// a band in chunk order. The chunking of a band depends only on its own length, so a band's
// result does not depend on which other bands share the call.
#include "common.hpp"
#include "kernels.hpp"

namespace dfl {

constexpr int KCMAX = 256;  // keys per chunk (16 pages); the runtime never plans more
constexpr int KSTEP = 64;   // keys per LDS buffer and softmax step
constexpr int RT = 2;       // 16-row query tiles per wavefront
constexpr int AW = 4;       // wavefronts per attention workgroup
constexpr int RPAD = AW * RT * 16;

// One 64-key step of the chunk in LDS.
//  k: K rows padded to HD + 8, stored in MFMA tile order: LDS row t*16 + m holds the key
//     that tile t's row m covers (kt_key below), so the 16 lanes reading one tile read 16
//     consecutive LDS rows and any 8 of them hit distinct banks.
//  v: the step's four V pages as stored ([d][16] per page) with the two 16-byte halves of a
//     row d swapped when bit 2 of d is set (vswz), so lanes reading rows d..d+7 of one half
//     hit distinct banks.
template <int HD>
struct AttnBuf {
  bf16 k[KSTEP][HD + 8];
  bf16 v[KSTEP / PAGE][HD][PAGE];
};

template <int HD>
struct AttnLds {
  AttnBuf<HD> buf[2];
  int pos[KCMAX];
  int page[KCMAX / PAGE];
};

// key (within a 64-key step) that row m of S^T tile t covers: tiles 2p and 2p+1 cover keys
// 32p..32p+31 such that lane (c, g) of the MFMA result holds keys 32p + 8g + 0..7 of query
// row c (4 from each tile)
__device__ __forceinline__ int kt_key(int t, int m) { return (t >> 1) * 32 + (m >> 2) * 8 + (t & 1) * 4 + (m & 3); }
// inverse: LDS row of a key
__device__ __forceinline__ int key_row(int kl) {
  const int w = kl & 31;
  return ((kl >> 5) * 2 + ((w >> 2) & 1)) * 16 + (w >> 3) * 4 + (w & 3);
}
__device__ __forceinline__ int vswz(int d) { return (d >> 2) & 1; }

// the 16-byte pieces of one step each thread carries from HBM to LDS
template <int HD>
struct StepRegs {
  static constexpr int PIECES = KSTEP * HD / 8;          // per K (and per V)
  static constexpr int PER_T = (PIECES + AW * 64 - 1) / (AW * 64);
  u32x4 k[PER_T], v[PER_T];
};

template <int HD>
__device__ __forceinline__ void step_load(StepRegs<HD>& rg, const AttnLds<HD>& sm, const bf16* lpool,
                                          size_t pl, int kvh, int nkv, int step) {
  constexpr int P8 = HD / 8;
#pragma unroll
  for (int u = 0; u < StepRegs<HD>::PER_T; ++u) {
    const int pc = u * AW * 64 + threadIdx.x;          // piece of this step
    if (pc < StepRegs<HD>::PIECES) {
      const int kl = pc / P8, d8 = pc % P8;              // key of the step, 8-element slice
      const int pg = sm.page[step * (KSTEP / PAGE) + (kl >> 4)];
      rg.k[u] = *reinterpret_cast<const u32x4*>(lpool + (size_t)pg * pl + ((size_t)kvh * PAGE + (kl & 15)) * HD + d8 * 8);
      const int vp = pc / (HD * 2), vo = pc % (HD * 2);   // V: page of the step, 16-byte slice
      const int pgv = sm.page[step * (KSTEP / PAGE) + vp];
      rg.v[u] = *reinterpret_cast<const u32x4*>(lpool + (size_t)pgv * pl + (size_t)(nkv + kvh) * HD * PAGE + vo * 8);
    }
  }
}

template <int HD>
__device__ __forceinline__ void step_store(AttnBuf<HD>& b, const StepRegs<HD>& rg) {
  constexpr int P8 = HD / 8;
#pragma unroll
  for (int u = 0; u < StepRegs<HD>::PER_T; ++u) {
    const int pc = u * AW * 64 + threadIdx.x;
    if (pc < StepRegs<HD>::PIECES) {
      const int kl = pc / P8, d8 = pc % P8;
      *reinterpret_cast<u32x4*>(&b.k[key_row(kl)][d8 * 8]) = rg.k[u];
      const int vp = pc / (HD * 2), d = (pc % (HD * 2)) >> 1, h = pc & 1;
      *reinterpret_cast<u32x4*>(&b.v[vp][d][(h ^ vswz(d)) * 8]) = rg.v[u];
    }
  }
}

template <int HD, bool WIN>
__global__ __launch_bounds__(AW * 64) void k_block_attn(const bf16* __restrict__ Q,
                                                        const bf16* __restrict__ Q_lo,
                                                        const Band* __restrict__ bands, int n_bands,
                                                        int gamma, int nh, KvGeom g, int layer, int sw,
                                                        int window, float scale_log2,
                                                        float* __restrict__ part_o,
                                                        float* __restrict__ part_ml) {
  constexpr int NS = HD / 32;
  constexpr int ND = HD / 16;
  __shared__ __attribute__((aligned(16))) AttnLds<HD> sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, grp = lane >> 4;
  const int kvh = blockIdx.y;
  const int nkv = g.nkv;
  const int G = nh / nkv;
  const int cg = blockIdx.x;
  int b = 0;
  while (b + 1 < n_bands && cg >= bands[b + 1].base[sw]) ++b;
  const int seq = bands[b].seq, C = bands[b].kv_len, qpos0 = bands[b].q_pos;
  const int ch = cg - bands[b].base[sw];
  const int kend = C + gamma;
  const int k0 = bands[b].kstart[sw] + ch * bands[b].ck[sw];   // page aligned
  const int k1 = min(k0 + bands[b].ck[sw], kend);
  const int npg = (k1 - k0 + PAGE - 1) / PAGE;                 // pages holding keys of the chunk
  const int nsteps = (k1 - k0 + KSTEP - 1) / KSTEP;
  const int nst = nsteps * (KSTEP / PAGE);                     // pages staged: whole steps
  const int R = gamma * G;
  const size_t pl = page_layer_elems(nkv, HD);
  const bf16* lpool = g.pool + (size_t)layer * g.num_pages * pl;

  // page ids and stamped positions of the chunk. Pages of a step past the chunk's end are
  // the zeroed sentinel page 0, so every value the MFMAs read is finite (masked keys then
  // contribute exactly zero).
  if (threadIdx.x < nst)
    sm.page[threadIdx.x] = threadIdx.x < npg ? g.bt[(size_t)seq * g.per_seq + (k0 >> 4) + threadIdx.x] : 0;
  __syncthreads();
  if (WIN)
    for (int kl = threadIdx.x; kl < nst * PAGE; kl += AW * 64) sm.pos[kl] = g.kpos[(size_t)sm.page[kl >> 4] * PAGE + (kl & 15)];

  StepRegs<HD> rg;
  step_load<HD>(rg, sm, lpool, pl, kvh, nkv, 0);

  // this wave's query rows: tile rt holds rows r = (wave * RT + rt) * 16 + c, i.e. block
  // row r % gamma of query head r / gamma (of this kv head's group)
  const bool wave_active = wave * RT * 16 < R;
  bf16x8 qb[RT][NS], ql[RT][NS];
  int qpos[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = (wave * RT + rt) * 16 + c;
    const bool rv = r < R;
    const int i = rv ? r % gamma : 0, hq = rv ? r / gamma : 0;
    const size_t qo = ((size_t)(b * gamma + i) * nh + kvh * G + hq) * HD + grp * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qb[rt][s] = ld8(Q + qo + s * 32);
      ql[rt][s] = ld8(Q_lo + qo + s * 32);
    }
    qpos[rt] = qpos0 + i;
  }
  float m_run[RT], l_run[RT];
  f32x4 o[RT][ND];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  step_store<HD>(sm.buf[0], rg);
  __syncthreads();

  for (int st = 0; st < nsteps; ++st) {
    // the next step's pieces are in flight while this one is computed
    if (st + 1 < nsteps) step_load<HD>(rg, sm, lpool, pl, kvh, nkv, st + 1);
    const AttnBuf<HD>& bf = sm.buf[st & 1];
    const int kt = st * KSTEP;
    const int lim = k1 - k0 - kt;   // keys of this step that exist
    if (wave_active) {
      // S^T = K Q^T: per tile and row tile, the hi and lo query terms accumulate in separate
      // chains, so consecutive MFMAs are independent
      f32x4 sh[RT][4], sl[RT][4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sh[rt][t] = sl[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&bf.k[t * 16 + c][s * 32 + grp * 8]));
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            sh[rt][t] = mfma16(a, qb[rt][s], sh[rt][t]);
            sl[rt][t] = mfma16(a, ql[rt][s], sl[rt][t]);
          }
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        // lane (c, grp) holds keys p*32 + grp*8 + 0..7 (p = 0, 1) of row c: element e is key
        // (e/8)*32 + grp*8 + e%8, from tile 2*(e/8) + (e/4)%2, slot e%4
        float sv[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kl = (e >> 3) * 32 + grp * 8 + (e & 7);
          const int t = (e >> 3) * 2 + ((e >> 2) & 1);
          const float x = (sh[rt][t][e & 3] + sl[rt][t][e & 3]) * scale_log2;
          bool ok = kl < lim;
          if (WIN) ok = ok & (qpos[rt] - sm.pos[kt + kl] < window);
          sv[e] = ok ? x : -INFINITY;
          tmax = fmaxf(tmax, sv[e]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run[rt], tmax);
        // rescale the running output only when some row's maximum moved
        if (__any(m_new > m_run[rt])) {
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[rt] - m_new);
          l_run[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) o[rt][dt] *= alpha;
        }
        m_run[rt] = m_new;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sv[e] = (sv[e] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sv[e] - m_new);
          l_run[rt] += sv[e];
        }
        // O^T += V^T P^T over the two 32-key halves
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
          const bf16x8 pb = pack8(sv + ps * 8);
          const int kl = ps * 32 + grp * 8;
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            const int d = dt * 16 + c;
            const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                &bf.v[kl >> 4][d][(((kl & 15) >> 3) ^ vswz(d)) * 8]));
            o[rt][dt] = mfma16(a, pb, o[rt][dt]);
          }
        }
      }
    }
    if (st + 1 < nsteps) step_store<HD>(sm.buf[(st + 1) & 1], rg);
    __syncthreads();
  }

  const size_t item = (size_t)cg * nkv + kvh;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float lt = l_run[rt];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int r = (wave * RT + rt) * 16 + c;
    if (r < R) {
      float* po = part_o + (item * RPAD + r) * HD + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[rt][dt];
      if (grp == 0) {
        part_ml[(item * RPAD + r) * 2 + 0] = m_run[rt];
        part_ml[(item * RPAD + r) * 2 + 1] = lt;
      }
    }
  }
}

hipError_t launch_block_attn(const bf16* Q, const bf16* Q_lo, const Band* bands_dev, int n_bands, int total_chunks,
                             int gamma, int nh, KvGeom g, int layer, int sw, int window,
                             float scale_log2, float* part_o, float* part_ml, hipStream_t st) {
  const int G = nh / g.nkv;
  if (gamma * G > RPAD) return hipErrorInvalidValue;
  dim3 grid(total_chunks, g.nkv);
#define DFL_ATTN(HDV, W) (void)launch(k_block_attn<HDV, W>, grid, AW * 64, 0, st, Q, Q_lo, bands_dev, n_bands, gamma, nh, g, layer, sw, window, scale_log2, part_o, part_ml)
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

// merge a band's chunks in chunk order: one workgroup per (band, kv head, 16 query rows);
// thread (row, 8-float slice of the head)
template <int HD>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const Band* __restrict__ bands, int gamma,
                                                      int nh, int nkv, int sw, int rpad,
                                                      bf16* __restrict__ out,
                                                      bf16* __restrict__ out_lo) {
  constexpr int DC = HD / 8;
  const int b = blockIdx.x, kvh = blockIdx.y;
  const int rl = threadIdx.x / DC, dc = threadIdx.x % DC;
  const int r = blockIdx.z * 16 + rl;
  const int G = nh / nkv;
  if (rl >= 16 || r >= gamma * G) return;
  const int i = r % gamma, hq = r / gamma;
  const int nch = bands[b].nch[sw], base = bands[b].base[sw];
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) {
    const size_t item = (size_t)(base + c) * nkv + kvh;
    M = fmaxf(M, part_ml[(item * rpad + r) * 2]);
  }
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll 4
  for (int c = 0; c < nch; ++c) {
    const size_t item = (size_t)(base + c) * nkv + kvh;
    const float mc = part_ml[(item * rpad + r) * 2];
    const float lc = part_ml[(item * rpad + r) * 2 + 1];
    const f32x4* po = reinterpret_cast<const f32x4*>(part_o + (item * rpad + r) * HD + dc * 8);
    const f32x4 o0 = po[0], o1 = po[1];
    const float w = (mc == -INFINITY) ? 0.f : exp2f(mc - M);
    L += w * lc;
    a0 += w * o0;
    a1 += w * o1;
  }
  const float inv = 1.f / L;
  const size_t o = ((size_t)(b * gamma + i) * nh + kvh * G + hq) * HD + dc * 8;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    split_bf16(a0[e] * inv, out[o + e], out_lo[o + e]);
    split_bf16(a1[e] * inv, out[o + 4 + e], out_lo[o + 4 + e]);
  }
}

hipError_t launch_attn_combine(const float* part_o, const float* part_ml, const Band* bands_dev,
                               int n_bands, int gamma, int nh, int nkv, int hd, int sw,
                               bf16* out, bf16* out_lo, hipStream_t st) {
  const int G = nh / nkv;
  const int rpad = RPAD;
  dim3 grid(n_bands, nkv, (gamma * G + 15) / 16);
  switch (hd) {
    case 32: (void)launch(k_attn_combine<32>, grid, 256, 0, st, part_o, part_ml, bands_dev, gamma, nh, nkv, sw, rpad, out, out_lo); break;
    case 64: (void)launch(k_attn_combine<64>, grid, 256, 0, st, part_o, part_ml, bands_dev, gamma, nh, nkv, sw, rpad, out, out_lo); break;
    case 128: (void)launch(k_attn_combine<128>, grid, 256, 0, st, part_o, part_ml, bands_dev, gamma, nh, nkv, sw, rpad, out, out_lo); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dfl
