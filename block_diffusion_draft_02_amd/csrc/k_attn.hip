// Non-causal paged GQA block attention (memra_engine/dflash.rs, DflashDraft::forward_round:
// every block query sees every context key and every block key; scale 1/sqrt(head_dim);
// sliding layers additionally hide keys with q_pos - k_pos >= window).
//
// Work split: one workgroup per (band, kv head, key chunk). Its four wavefronts own the
// band's gamma * G query rows of that kv head (G = query heads per kv head), 16 or 32 rows
// each, and walk the chunk 32 keys at a time:
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

template <int HD, int RT>
__global__ __launch_bounds__(256) void k_block_attn(const bf16* __restrict__ Q,
                                                    const Band* __restrict__ bands, int n_bands,
                                                    int gamma, int nh, KvGeom g, int layer, int sw,
                                                    int window, float scale_log2,
                                                    float* __restrict__ part_o,
                                                    float* __restrict__ part_ml) {
  constexpr int NS = HD / 32;
  constexpr int ND = HD / 16;
  constexpr int RPAD = 4 * RT * 16;
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
  const int k0 = bands[b].kstart[sw] + ch * bands[b].ck[sw];
  const int k1 = min(k0 + bands[b].ck[sw], kend);
  const int R = gamma * G;
  const int* btrow = g.bt + (size_t)seq * g.per_seq;
  const size_t pl = page_layer_elems(nkv, HD);
  const bf16* lpool = g.pool + (size_t)layer * g.num_pages * pl;

  bf16x8 qb[RT][NS];
  int qpos[RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    const int r = (wave * RT + j) * 16 + c;
    const bool rv = r < R;
    const int i = rv ? r % gamma : 0, hq = rv ? r / gamma : 0;
    const bf16* qp = Q + ((size_t)(b * gamma + i) * nh + kvh * G + hq) * HD + grp * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) qb[j][s] = ld8(qp + s * 32);
    qpos[j] = qpos0 + i;
  }
  float m_run[RT], l_run[RT];
  f32x4 o[RT][ND];
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int kt = k0; kt < k1; kt += 32) {
    f32x4 sacc[RT][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = kt + (c >> 2) * 8 + t * 4 + (c & 3);
      const int page = key < k1 ? btrow[key >> 4] : 0;
      const bf16* kp = lpool + (size_t)page * pl + ((size_t)kvh * PAGE + (key & 15)) * HD + grp * 8;
#pragma unroll
      for (int j = 0; j < RT; ++j) sacc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 a = ld8(kp + s * 32);
#pragma unroll
        for (int j = 0; j < RT; ++j) sacc[j][t] = mfma16(a, qb[j][s], sacc[j][t]);
      }
    }
    // this lane now holds, for query row c of every row tile, keys kbase + 0..7
    const int kbase = kt + grp * 8;
    const int pg8 = kbase < k1 ? btrow[kbase >> 4] : 0;
    int kp8[8];
    if (window > 0) {
      const int* kq = g.kpos + (size_t)pg8 * PAGE + (kbase & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) kp8[e] = kq[e];
    }
    bf16x8 pb[RT];
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      float sv[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kbase + e;
        bool ok = key < k1;
        if (window > 0) ok = ok && (qpos[j] - kp8[e] < window);
        sv[e] = ok ? sacc[j][e >> 2][e & 3] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[e]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run[j], tmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run[j] - m_new);
      float p[8];
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = (sv[e] == -INFINITY) ? 0.f : exp2f(sv[e] - m_new);
        ps += p[e];
      }
      l_run[j] = l_run[j] * alpha + ps;
      m_run[j] = m_new;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) o[j][dt] *= alpha;
      pb[j] = pack8(p);
    }
    const bf16* vp = lpool + (size_t)pg8 * pl + (size_t)(nkv + kvh) * HD * PAGE + (kbase & 15);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const bf16x8 a = ld8(vp + (size_t)(dt * 16 + c) * PAGE);
#pragma unroll
      for (int j = 0; j < RT; ++j) o[j][dt] = mfma16(a, pb[j], o[j][dt]);
    }
  }

  const size_t item = (size_t)cg * nkv + kvh;
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    float lt = l_run[j];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int r = (wave * RT + j) * 16 + c;
    if (r >= R) continue;
    float* po = part_o + (item * RPAD + r) * HD + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[j][dt];
    if (grp == 0) {
      part_ml[(item * RPAD + r) * 2 + 0] = m_run[j];
      part_ml[(item * RPAD + r) * 2 + 1] = lt;
    }
  }
}

static int attn_rt(int gamma, int G) { return gamma * G <= 64 ? 1 : 2; }

hipError_t launch_block_attn(const bf16* Q, const Band* bands_dev, int n_bands, int total_chunks,
                             int gamma, int nh, KvGeom g, int layer, int sw, int window,
                             float scale_log2, float* part_o, float* part_ml, hipStream_t st) {
  const int G = nh / g.nkv;
  if (gamma * G > 128) return hipErrorInvalidValue;
  dim3 grid(total_chunks, g.nkv);
  const int rt = attn_rt(gamma, G);
#define DFL_ATTN(HDV, RTV)                                                                   \
  k_block_attn<HDV, RTV><<<grid, 256, 0, st>>>(Q, bands_dev, n_bands, gamma, nh, g, layer, sw, \
                                               window, scale_log2, part_o, part_ml)
  if (g.hd == 128) { if (rt == 1) DFL_ATTN(128, 1); else DFL_ATTN(128, 2); }
  else if (g.hd == 64) { if (rt == 1) DFL_ATTN(64, 1); else DFL_ATTN(64, 2); }
  else if (g.hd == 32) { if (rt == 1) DFL_ATTN(32, 1); else DFL_ATTN(32, 2); }
  else return hipErrorInvalidValue;
#undef DFL_ATTN
  return hipGetLastError();
}

// one wavefront per (band, kv head, query row): merge the band's chunks in chunk order
template <int HD>
__global__ __launch_bounds__(64) void k_attn_combine(const float* __restrict__ part_o,
                                                     const float* __restrict__ part_ml,
                                                     const Band* __restrict__ bands, int gamma,
                                                     int nh, int nkv, int sw, int rpad,
                                                     bf16* __restrict__ out) {
  const int b = blockIdx.x, kvh = blockIdx.y, r = blockIdx.z, l = threadIdx.x;
  const int G = nh / nkv;
  const int i = r % gamma, hq = r / gamma;
  const int nch = bands[b].nch[sw], base = bands[b].base[sw];
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) {
    const size_t item = (size_t)(base + c) * nkv + kvh;
    M = fmaxf(M, part_ml[(item * rpad + r) * 2]);
  }
  constexpr int E = HD > 64 ? HD / 64 : 1;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float L = 0.f;
  for (int c = 0; c < nch; ++c) {
    const size_t item = (size_t)(base + c) * nkv + kvh;
    const float mc = part_ml[(item * rpad + r) * 2];
    const float w = (mc == -INFINITY) ? 0.f : exp2f(mc - M);
    L += w * part_ml[(item * rpad + r) * 2 + 1];
    const float* po = part_o + (item * rpad + r) * HD;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = l + 64 * e;
      if (d < HD) acc[e] += w * po[d];
    }
  }
  const float inv = 1.f / L;
  bf16* o = out + ((size_t)(b * gamma + i) * nh + kvh * G + hq) * HD;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int d = l + 64 * e;
    if (d < HD) o[d] = f2bf(acc[e] * inv);
  }
}

hipError_t launch_attn_combine(const float* part_o, const float* part_ml, const Band* bands_dev,
                               int n_bands, int gamma, int nh, int nkv, int hd, int sw,
                               bf16* out, hipStream_t st) {
  const int G = nh / nkv;
  const int rpad = 4 * attn_rt(gamma, G) * 16;
  dim3 grid(n_bands, nkv, gamma * G);
  switch (hd) {
    case 32: k_attn_combine<32><<<grid, 64, 0, st>>>(part_o, part_ml, bands_dev, gamma, nh, nkv, sw, rpad, out); break;
    case 64: k_attn_combine<64><<<grid, 64, 0, st>>>(part_o, part_ml, bands_dev, gamma, nh, nkv, sw, rpad, out); break;
    case 128: k_attn_combine<128><<<grid, 64, 0, st>>>(part_o, part_ml, bands_dev, gamma, nh, nkv, sw, rpad, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dfl
