// Non-causal paged GQA block attention (memra_engine/dflash.rs, DflashDraft::forward_round:
// every block query sees every context key and every block key; scale 1/sqrt(head_dim);
// sliding layers additionally hide keys with q_pos - k_pos >= window).
//
// Work split: one workgroup per (band, kv head, key chunk of at most 256 keys). The
// workgroup first stages the chunk's K rows, V pages and key positions in LDS with every
// load in flight at once; its four wavefronts then own the band's gamma * G query rows of
// that kv head (G = query heads per kv head), 16 or 32 rows each, and walk the chunk 32 keys
// at a time:
//   S^T = K Q^T   two 16x16x32 MFMA tiles per 32 keys; the key order inside the tiles is
//                 permuted so that every lane ends up holding 8 consecutive keys of one row
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

// The chunk's keys in LDS: K rows padded to HD + 8 (1 KB + 16 B rows keep the MFMA operand
// reads of any 8 consecutive lanes on distinct banks), V pages as stored ([d][16] per page),
// the stamped position of every key, and the chunk's physical pages.
template <int HD>
struct AttnLds {
  bf16 k[KCMAX][HD + 8];
  bf16 v[KCMAX / PAGE][HD][PAGE];
  int pos[KCMAX];
  int page[KCMAX / PAGE];
};

constexpr int AW = 8;       // wavefronts per attention workgroup, 16 query rows each
constexpr int RPAD = AW * 16;

template <int HD>
__global__ __launch_bounds__(AW * 64) void k_block_attn(const bf16* __restrict__ Q,
                                                        const bf16* __restrict__ Q_lo,
                                                        const Band* __restrict__ bands, int n_bands,
                                                        int gamma, int nh, KvGeom g, int layer, int sw,
                                                        int window, float scale_log2,
                                                        float* __restrict__ part_o,
                                                        float* __restrict__ part_ml) {
  constexpr int NS = HD / 32;
  constexpr int ND = HD / 16;
  constexpr int P8 = HD / 8;  // 16-byte pieces per K row
  constexpr int NT = AW * 64;
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
  const int nst = (k1 - k0 + 63) / 64 * 4;                     // pages staged: whole 64-key steps
  const int R = gamma * G;
  const size_t pl = page_layer_elems(nkv, HD);
  const bf16* lpool = g.pool + (size_t)layer * g.num_pages * pl;

  // ---- stage the chunk: page ids, then every K row, V page and position at once. Pages of
  // a step past the chunk's end are the zeroed sentinel page 0, so every value the MFMAs
  // read is finite (masked keys then contribute exactly zero).
  if (threadIdx.x < nst)
    sm.page[threadIdx.x] = threadIdx.x < npg ? g.bt[(size_t)seq * g.per_seq + (k0 >> 4) + threadIdx.x] : 0;
  __syncthreads();
  {
    const int nk = nst * PAGE;
    const int pieces = nk * P8;          // K pieces; V has the same count
    for (int base = 0; base < pieces; base += NT * 8) {
      u32x4 kr[8], vr[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pc = base + u * NT + threadIdx.x;
        if (pc < pieces) {
          const int kl = pc / P8, d8 = pc % P8;
          kr[u] = *reinterpret_cast<const u32x4*>(lpool + (size_t)sm.page[kl >> 4] * pl +
                                                  ((size_t)kvh * PAGE + (kl & 15)) * HD + d8 * 8);
          const int vp = pc / (HD * 2), vo = pc % (HD * 2);
          vr[u] = *reinterpret_cast<const u32x4*>(lpool + (size_t)sm.page[vp] * pl +
                                                  (size_t)(nkv + kvh) * HD * PAGE + vo * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pc = base + u * NT + threadIdx.x;
        if (pc < pieces) {
          const int kl = pc / P8, d8 = pc % P8;
          *reinterpret_cast<u32x4*>(&sm.k[kl][d8 * 8]) = kr[u];
          *reinterpret_cast<u32x4*>(&sm.v[0][0][0] + (size_t)pc * 8) = vr[u];
        }
      }
    }
    if (window > 0)
      for (int kl = threadIdx.x; kl < nk; kl += NT) sm.pos[kl] = g.kpos[(size_t)sm.page[kl >> 4] * PAGE + (kl & 15)];
  }

  // this wave's 16 query rows: r = wave * 16 + c (block row r % gamma, head r / gamma)
  const int r = wave * 16 + c;
  const bool rv = r < R;
  const bool wave_active = wave * 16 < R;
  bf16x8 qb[NS], ql[NS];
  int qpos;
  {
    const int i = rv ? r % gamma : 0, hq = rv ? r / gamma : 0;
    const size_t qo = ((size_t)(b * gamma + i) * nh + kvh * G + hq) * HD + grp * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qb[s] = ld8(Q + qo + s * 32);
      ql[s] = ld8(Q_lo + qo + s * 32);
    }
    qpos = qpos0 + i;
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  if (wave_active) {
    for (int kt = 0; kt < k1 - k0; kt += 64) {
      // S^T for 64 keys: MFMA tile t covers keys (t/2)*32 + (m/4)*8 + (t%2)*4 + m%4 for its
      // row m, so lane (c, grp) ends up with keys kt + p*32 + grp*8 + 0..7 (p = 0, 1) of row c
      f32x4 sacc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kl = kt + (t >> 1) * 32 + (c >> 2) * 8 + (t & 1) * 4 + (c & 3);
        sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.k[kl][s * 32 + grp * 8]));
          sacc[t] = mfma16(a, qb[s], sacc[t]);
          sacc[t] = mfma16(a, ql[s], sacc[t]);
        }
      }
      float sv[16];
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kl = kt + (e >> 3) * 32 + grp * 8 + (e & 7);
        bool ok = k0 + kl < k1;
        if (window > 0) ok = ok && (qpos - sm.pos[kl] < window);
        sv[e] = ok ? sacc[(e >> 3) * 2 + ((e >> 2) & 1)][e & 3] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[e]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax);
      // rescale the running output only when some row's maximum moved
      if (__any(m_new > m_run)) {
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) o[dt] *= alpha;
      }
      m_run = m_new;
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = (sv[e] == -INFINITY) ? 0.f : exp2f(sv[e] - m_new);
        l_run += p[e];
      }
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) {
        const bf16x8 pb = pack8(p + ps * 8);
        const int kl = kt + ps * 32 + grp * 8;
        const bf16* vp = &sm.v[kl >> 4][0][kl & 15];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vp + (size_t)(dt * 16 + c) * PAGE));
          o[dt] = mfma16(a, pb, o[dt]);
        }
      }
    }
  }

  float lt = l_run;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (!rv) return;
  const size_t item = (size_t)cg * nkv + kvh;
  float* po = part_o + (item * RPAD + r) * HD + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[dt];
  if (grp == 0) {
    part_ml[(item * RPAD + r) * 2 + 0] = m_run;
    part_ml[(item * RPAD + r) * 2 + 1] = lt;
  }
}

hipError_t launch_block_attn(const bf16* Q, const bf16* Q_lo, const Band* bands_dev, int n_bands, int total_chunks,
                             int gamma, int nh, KvGeom g, int layer, int sw, int window,
                             float scale_log2, float* part_o, float* part_ml, hipStream_t st) {
  const int G = nh / g.nkv;
  if (gamma * G > RPAD) return hipErrorInvalidValue;
  dim3 grid(total_chunks, g.nkv);
  switch (g.hd) {
    case 128: (void)launch(k_block_attn<128>, grid, AW * 64, 0, st, Q, Q_lo, bands_dev, n_bands, gamma, nh, g, layer, sw, window, scale_log2, part_o, part_ml); break;
    case 64: (void)launch(k_block_attn<64>, grid, AW * 64, 0, st, Q, Q_lo, bands_dev, n_bands, gamma, nh, g, layer, sw, window, scale_log2, part_o, part_ml); break;
    case 32: (void)launch(k_block_attn<32>, grid, AW * 64, 0, st, Q, Q_lo, bands_dev, n_bands, gamma, nh, g, layer, sw, window, scale_log2, part_o, part_ml); break;
    default: return hipErrorInvalidValue;
  }
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
