// LDS-tiled 256 x 256 BF16 MFMA GEMM for the context append (thousands of rows), fed by a
// ring of global->LDS stages.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace dfl {

constexpr int TB_M = 256, TB_N = 256;  // output tile of a workgroup
constexpr int TK = 32;                 // depth of one MFMA step
constexpr int T_WAVES = 8;             // 4 row quarters x 2 column halves: a wave owns 64 x 128
constexpr int T_KS_MAX = 4;            // k splits at most

// The ring: with the lo term (SPLIT) a stage is one 32-deep step (48 KB) and the ring three
// stages; an exact activation's stage is two steps deep (64 KB) and the ring two stages, so
// its barrier and waits come once per 64 MFMAs a wave, as with the lo term.
template <bool SPLIT>
struct TiledShape {
  static constexpr int TKS = SPLIT ? 32 : 64;   // k depth of a stage
  static constexpr int NST = SPLIT ? 3 : 2;     // stages in the ring
  static constexpr int UPR = TKS / 8;           // 16-byte units of a stage row
  static constexpr int NP = UPR / 2;            // 1 KB DMA pieces of one operand a wave brings per stage
};

// one stage: the A rows (hi and, with SPLIT, lo) and the W rows of its k range, TKS * 2 bytes
// a row; row r's 16-byte unit u sits at unit u ^ ((r >> 1) & (UPR - 1)), so the 16 lanes an
// LDS cycle serves (rows of a 16-row fragment, one unit) hit distinct 16-byte bank groups
template <bool SPLIT>
struct TiledStage {
  bf16 a[TB_M * TiledShape<SPLIT>::TKS];
  bf16 al[SPLIT ? TB_M * TiledShape<SPLIT>::TKS : 8];
  bf16 w[TB_N * TiledShape<SPLIT>::TKS];
};

// s_waitcnt with vmcnt <= N (vmcnt[3:0] | vmcnt[5:4] << 14; expcnt and lgkmcnt left at maximum)
#define DFL_GEMM_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))

// k splits: from (N, K) alone, never from the row count, so that a row's result does not
// depend on how rows are grouped into launches. A narrow output (few 256-column tiles) splits
// its K in two or four so that a 2048-row launch still has about a chip's worth of workgroups.
// Each split is a whole number of the deeper (64) stages.
int gemm_tiled_splits(int N, int K) {
  const int tiles = (APPEND_ROWS / TB_M) * ((N + TB_N - 1) / TB_N);
  int ks = 1;
  while (ks < T_KS_MAX && tiles * ks * 2 <= 256 && K % (TiledShape<false>::TKS * ks * 2) == 0) ks *= 2;
  return ks;
}

// the fused K/V epilogue's inputs (launch_gemm_tiled_kv)
struct KvEpi {
  const long long* slots;   // [M] pool slot of each row
  const float2* cs;         // [M][hd / 2] the rows' RoPE (cos, sin)
  const bf16* kn_all;       // [L][hd] k_norm weights
  float eps, mscale;
  KvGeom g;
};

// lane l's v from lane l ^ X (X < 32): ds_swizzle's bit mode, and mask 0x1f
template <int X>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (X << 10) | 0x1f));
}

__device__ __forceinline__ long long shfl64(long long v, int src) {
  const int lo = __shfl((int)(unsigned long long)v, src), hi = __shfl((int)((unsigned long long)v >> 32), src);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// The K/V epilogue of one wave's 64 x 128 piece of a tile: rows R0 .. R0+63 (R0 = m0 + 64 wm),
// columns = HW = 128 / HD whole heads of one layer's K or V block. The wave's region is 16 KB
// of LDS no other wave touches; it carries the values to the pool (V in two passes of 64
// columns).
// K: x = 0 + the GEMM's result; the head's sum of squares (over j in this lane, then over the
// 16 lanes of the row, which all end with the same sum); k_norm; RoPE on the pairs (d, d +
// HD/2), which sit in this lane's j-blocks jj and jj + JH/2; times mscale; staged in LDS as
// each is made, then 16-byte stores along the page's [key][d] rows (16 lanes a 256-byte row).
// V: bf16(0 + result), staged [d][key] with the keys shifted by the first row's page offset,
// so that a 16-key group is one page row: 16-byte stores where the group's 16 rows have
// consecutive slots starting a page, element stores elsewhere.
template <int HD>
__device__ __forceinline__ void kv_epilogue(f32x4 (&acc)[4][8], char* reg, int m0, int n0, int M, int wm, int wn,
                                            int lane, const KvEpi& ep) {
  constexpr int HALF = HD / 2, JH = HD / 16, HW = 128 / HD;
  const KvGeom& g = ep.g;
  const int c = lane & 15, gq = lane >> 4;
  const int kvd = g.nkv * HD;
  const int blk = n0 / kvd;   // layer * 2 + (0 for K, 1 for V)
  const int layer = blk >> 1;
  const int head0 = (n0 - blk * kvd) / HD + wn * HW;
  const int R0 = m0 + wm * 64;
  const int nv = min(64, M - R0);   // rows of the wave that exist
  if (nv <= 0) return;
  const long long pl = (long long)page_layer_elems(g.nkv, HD);
  bf16* const lay = g.pool + (size_t)layer * g.num_pages * pl;
  const long long sl = lane < nv ? ep.slots[R0 + lane] : -1;
  if ((blk & 1) == 0) {
    // [64 rows][128 columns], 256-byte rows; 16-byte unit u of row r at u ^ 2 ((r >> 2) & 3), so
    // the four rows a 2-byte store instruction touches (4 apart) fall on distinct banks. This
    // lane's rows are 16 i + 4 gq + e, so its swizzle is 2 gq throughout: one address per
    // j-block, the row a constant offset.
    char* kb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kb[j] = reg + gq * 1024 + (2 * (j ^ gq) + (c >> 3)) * 16 + (c & 7) * 2;
    auto kst = [&](int i, int e, int j, bf16 v) { *reinterpret_cast<bf16*>(kb[j] + (i * 16 + e) * 256) = v; };
    const bf16* kn = ep.kn_all + (size_t)layer * HD;
    float w1[JH / 2], w2[JH / 2];
#pragma unroll
    for (int jj = 0; jj < JH / 2; ++jj) {
      w1[jj] = bf2f(kn[jj * 16 + c]);
      w2[jj] = bf2f(kn[HALF + jj * 16 + c]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = min(R0 + i * 16 + 4 * gq + e, M - 1);
        float2 cs[JH / 2];
#pragma unroll
        for (int jj = 0; jj < JH / 2; ++jj) cs[jj] = ep.cs[(size_t)m * HALF + jj * 16 + c];
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
          float x[JH];
          float ss = 0.f;
#pragma unroll
          for (int jj = 0; jj < JH; ++jj) {
            x[jj] = 0.f + acc[i][hh * JH + jj][e];
            ss += x[jj] * x[jj];
          }
          ss += swz_xor<1>(ss);
          ss += swz_xor<2>(ss);
          ss += swz_xor<4>(ss);
          ss += swz_xor<8>(ss);
          const float rs = rsqrtf(ss / (float)HD + ep.eps);
#pragma unroll
          for (int jj = 0; jj < JH / 2; ++jj) {
            const float a = x[jj] * (rs * w1[jj]), b = x[jj + JH / 2] * (rs * w2[jj]);
            const float cf = cs[jj].x, sf = cs[jj].y;
            const float y1 = a * cf - b * sf;
            const float y2 = b * cf + a * sf;
            kst(i, e, hh * JH + jj, f2bf(y1 * ep.mscale));
            kst(i, e, hh * JH + jj + JH / 2, f2bf(y2 * ep.mscale));
          }
        }
      }
      // one 16-row block at a time: hoisting more of the table loads runs out of registers
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 16 lanes a row: 16 bytes each, the row's 256 bytes
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int row = it * 4 + (lane >> 4), u = lane & 15;
      const long long slot = shfl64(sl, row);
      if (row < nv) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(reg + row * 256 + ((u ^ (2 * ((row >> 2) & 3))) * 16));
        const int col = u * 8;
        bf16* dst = lay + (slot >> 4) * pl + (size_t)(head0 + col / HD) * PAGE * HD + (int)(slot & (PAGE - 1)) * HD +
                    col % HD;
        *reinterpret_cast<u32x4*>(dst) = v;
      }
    }
    return;
  }
  // V: which rows continue their predecessor's slot, and the first row's offset in its page
  const long long prev = shfl64(sl, lane > 0 ? lane - 1 : 0);
  const unsigned long long cont = __ballot(lane > 0 && lane < nv && sl == prev + 1);
  const int off = (int)(shfl64(sl, 0) & (PAGE - 1));
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    // [64 columns][88 keys], 176-byte rows; key = off + row
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<bf16*>(reg + (jj * 16 + c) * 176 + (off + i * 16 + 4 * gq + e) * 2) =
              f2bf(0.f + acc[i][4 * p + jj][e]);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int a = 16 * q - off;   // the group's first row
      const long long s0 = shfl64(sl, max(a, 0));
      const bool whole = a >= 0 && a + 16 <= nv && ((cont >> (a + 1)) & 0x7FFFull) == 0x7FFFull && (s0 & (PAGE - 1)) == 0;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int col = cb * 32 + (lane >> 1), h8 = lane & 1;
        const int gcol = 64 * p + col;
        const size_t hoff = (size_t)(g.nkv + head0 + gcol / HD) * HD * PAGE + (size_t)(gcol % HD) * PAGE;
        if (whole) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(reg + col * 176 + (16 * q + 8 * h8) * 2);
          *reinterpret_cast<u32x4*>(lay + (s0 >> 4) * pl + hoff + 8 * h8) = v;
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int key = 16 * q + 8 * h8 + t, row = key - off;
            const long long s = shfl64(sl, min(max(row, 0), 63));
            if (row >= 0 && row < nv)
              lay[(s >> 4) * pl + hoff + (int)(s & (PAGE - 1))] = *reinterpret_cast<const bf16*>(reg + col * 176 + key * 2);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// C[z] = A W^T over k split z (plain fp32 results; within a split the sum over k runs in
// order, step by step, the hi then the lo term at every 32-deep step). One 8-wave workgroup
// per 256 x 256 tile and split, each wave 64 x 128 (four 16-row by eight 16-column MFMA
// tiles): per 32-deep step a wave reads 8 activation fragments (each hi and lo with SPLIT)
// and 8 weight fragments, and the workgroup brings 48 KB (32 KB without the lo term) into LDS
// for 256 x 256 x 32 products. The stages stream through the ring with the gfx950
// global->LDS 16-byte load: wave v brings an eighth of every operand of a stage, 1 KB an
// instruction, each lane choosing its source so that the LDS copy is swizzled. Stage j+NST-1
// is requested right after the barrier that ends stage j-1; a wave waits only for its own
// loads of stage j (one barrier per stage). Every stage issues the same loads (past the last
// one it re-reads the last into a stage nobody reads again), so the compiler sees one fixed
// count in flight, and the stages are separate LDS objects.
template <bool SPLIT, int EPI_HD>
__device__ __forceinline__ void gemm_tiled_wg(TiledStage<SPLIT>& st0, TiledStage<SPLIT>& st1, TiledStage<SPLIT>& st2,
                                              const bf16* __restrict__ A, const bf16* __restrict__ A_lo, int lda,
                                              int M, const bf16* __restrict__ W, int N, int K, int kps,
                                              float* __restrict__ C, int ldc, const KvEpi& ep) {
  using SH = TiledShape<SPLIT>;
  constexpr int TKS = SH::TKS, NST = SH::NST, UPR = SH::UPR, NP = SH::NP;
  constexpr int NI = NP * (SPLIT ? 3 : 2);   // DMA instructions per wave and stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * TB_M, n0 = blockIdx.x * TB_N;
  const int kb = blockIdx.z * kps;
  const int nk = kps / TKS;
  const int c = lane & 15, g = lane >> 4;
  // this wave's NP 1 KB pieces of each operand of a stage: LDS units P = (NP wave + h) * 64 +
  // lane, row P / UPR, source unit (P % UPR) ^ ((row >> 1) & (UPR - 1)); byte offsets (rows past
  // M or N repeat the last one; their results are never stored), loop-invariant
  uint32_t offA[NP], offW[NP];
#pragma unroll
  for (int h = 0; h < NP; ++h) {
    const int P = (NP * wave + h) * 64 + lane;
    const int r = P / UPR, u = (P % UPR) ^ ((r >> 1) & (UPR - 1));
    offA[h] = (uint32_t)((size_t)min(m0 + r, M - 1) * lda + u * 8) * 2u;
    offW[h] = (uint32_t)((size_t)min(n0 + r, N - 1) * K + u * 8) * 2u;
  }
  const bf16* srcA = A + kb;
  const bf16* srcAl = SPLIT ? A_lo + kb : A;
  const bf16* srcW = W + kb;
  auto issue = [&](TiledStage<SPLIT>& st, int j) {
    const int k = __builtin_amdgcn_readfirstlane(min(j, nk - 1) * TKS);
#pragma unroll
    for (int h = 0; h < NP; ++h) {
      const int o = (NP * wave + h) * 512;
      uint32_t va = offA[h], vw = offW[h];
      asm volatile("" : "+v"(va), "+v"(vw));
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(srcA + k) + va, &st.a[o], 16, 0, 0);
      if (SPLIT) __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(srcAl + k) + va, &st.al[o], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(srcW + k) + vw, &st.w[o], 16, 0, 0);
    }
  };
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the fragment of 32-deep step s of the stage
  auto frag = [&](const bf16* base, int r, int s) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + r * TKS + (((s * 4 + g) ^ ((r >> 1) & (UPR - 1))) * 8)));
  };
  auto mma = [&](const TiledStage<SPLIT>& st) {
#pragma unroll
    for (int s = 0; s < TKS / TK; ++s) {
      bf16x8 b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = frag(st.w, wn * 128 + j * 16 + c, s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a = frag(st.a, wm * 64 + i * 16 + c, s);
        const bf16x8 al = SPLIT ? frag(st.al, wm * 64 + i * 16 + c, s) : a;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          acc[i][j] = mfma16(a, b[j], acc[i][j]);
          if (SPLIT) acc[i][j] = mfma16(al, b[j], acc[i][j]);
        }
      }
    }
  };
  auto step = [&](int j, const TiledStage<SPLIT>& cur, TiledStage<SPLIT>& nxt) {
    DFL_GEMM_WAIT_VM(NI * (NST - 2));   // the next stages' loads may still be in flight
    __builtin_amdgcn_s_barrier();
    issue(nxt, j + NST - 1);
    if (j < nk) mma(cur);
  };
  issue(st0, 0);
  if constexpr (NST == 3) {
    issue(st1, 1);
    for (int j = 0; j < nk; j += 3) {
      step(j, st0, st2);
      step(j + 1, st1, st0);
      step(j + 2, st2, st1);
    }
  } else {
    for (int j = 0; j < nk; j += 2) {
      step(j, st0, st1);
      step(j + 1, st1, st0);
    }
  }
  DFL_GEMM_WAIT_VM(0);   // the loads past the last step land before the workgroup ends
  if constexpr (EPI_HD > 0) {
    // every wave is past its last read of the stages; each takes 16 KB of them
    __syncthreads();
    TiledStage<SPLIT>& sw = wave < 3 ? st0 : wave < 6 ? st1 : st2;
    char* reg = reinterpret_cast<char*>(&sw) + (wave % 3) * 16384;
    kv_epilogue<EPI_HD>(acc, reg, m0, n0, M, wm, wn, lane, ep);
    return;
  }
  float* Cz = C + (size_t)blockIdx.z * M * ldc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + wn * 128 + j * 16 + c;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 64 + i * 16 + 4 * g + e;
        if (m < M) Cz[(size_t)m * ldc + n] = acc[i][j][e];
      }
    }
  }
}

template <bool SPLIT, int EPI_HD>
__global__ __launch_bounds__(T_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_tiled(
    const bf16* __restrict__ A, const bf16* __restrict__ A_lo, int lda, int M, const bf16* __restrict__ W, int N,
    int K, int kps, float* __restrict__ C, int ldc, KvEpi ep) {
  __shared__ __attribute__((aligned(16))) TiledStage<SPLIT> st0, st1;
  if constexpr (TiledShape<SPLIT>::NST == 3) {
    __shared__ __attribute__((aligned(16))) TiledStage<SPLIT> st2;
    gemm_tiled_wg<SPLIT, EPI_HD>(st0, st1, st2, A, A_lo, lda, M, W, N, K, kps, C, ldc, ep);
  } else {
    gemm_tiled_wg<SPLIT, EPI_HD>(st0, st1, st1, A, A_lo, lda, M, W, N, K, kps, C, ldc, ep);
  }
}

hipError_t launch_gemm_tiled(const bf16* A, const bf16* A_lo, int lda, int M, const bf16* W, int N, int K, int ks,
                             float* C, int ldc, hipStream_t st) {
  const int tks = A_lo ? TiledShape<true>::TKS : TiledShape<false>::TKS;
  if (M <= 0 || N <= 0 || ks < 1 || ks > T_KS_MAX || K % (tks * ks) != 0 || (lda % 8) != 0 || ldc < N)
    return hipErrorInvalidValue;
  // the DMA offsets are 32-bit byte offsets from the operands' bases
  if ((size_t)M * lda * 2 >= (1ull << 32) || (size_t)N * K * 2 >= (1ull << 32)) return hipErrorInvalidValue;
  dim3 grid((N + TB_N - 1) / TB_N, (M + TB_M - 1) / TB_M, ks);
  const int kps = K / ks;
  const KvEpi none{};
  if (A_lo)
    (void)launch(k_gemm_tiled<true, 0>, grid, T_WAVES * 64, 0, st, A, A_lo, lda, M, W, N, K, kps, C, ldc, none);
  else
    (void)launch(k_gemm_tiled<false, 0>, grid, T_WAVES * 64, 0, st, A, A_lo, lda, M, W, N, K, kps, C, ldc, none);
  return hipGetLastError();
}

bool gemm_tiled_kv_fusable(int N, int nkv, int hd) {
  if (hd != 32 && hd != 64 && hd != 128) return false;
  const int kvd = nkv * hd;
  return kvd % TB_N == 0 && N % (2 * kvd) == 0;
}

hipError_t launch_gemm_tiled_kv(const bf16* A, const bf16* A_lo, int lda, int M, const bf16* W, int N, int K,
                                const bf16* k_norm_all, float eps, float mscale, const long long* slots,
                                const float2* cs, KvGeom g, hipStream_t st) {
  if (M <= 0 || !A_lo || !gemm_tiled_kv_fusable(N, g.nkv, g.hd) || K % TiledShape<true>::TKS != 0 || (lda % 8) != 0)
    return hipErrorInvalidValue;
  if ((size_t)M * lda * 2 >= (1ull << 32) || (size_t)N * K * 2 >= (1ull << 32)) return hipErrorInvalidValue;
  const KvEpi ep{slots, cs, k_norm_all, eps, mscale, g};
  dim3 grid(N / TB_N, (M + TB_M - 1) / TB_M, 1);
#define DFL_TKV(HDV) (void)launch(k_gemm_tiled<true, HDV>, grid, T_WAVES * 64, 0, st, A, A_lo, lda, M, W, N, K, K, (float*)nullptr, 0, ep)
  switch (g.hd) {
    case 32: DFL_TKV(32); break;
    case 64: DFL_TKV(64); break;
    default: DFL_TKV(128); break;
  }
#undef DFL_TKV
  return hipGetLastError();
}

}  // namespace dfl
