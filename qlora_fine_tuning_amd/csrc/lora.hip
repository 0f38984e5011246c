// Rank-r LoRA side-path kernels for gfx950 (HBM-bound "skinny" products).
//
// The chained-matmul bracketing of the Mistral benchmark page (items 10-11,
// "manual autograd") puts the rank-r product first: X A^T and dY B are
// [m][r] and cheap; the LoRA weight gradients dA = s T^T X and dB = s dY^T U
// are reductions over tokens of one big operand against an [m][r] one. All of
// these read one large bf16 operand once (X, dY, H, dg|du: 2 B per element)
// and are bound by HBM bandwidth, not by arithmetic.
//
//  rowdot     : U = G L^T  ([M][K] x [R][K]^T -> [M][R]) on MFMA 16x16x32;
//               64-row x 128-column tiles of G and L reach LDS by direct
//               loads in a 3-deep ring; K is split over blocks and the
//               partials are summed in a fixed order by a finish pass, which
//               also emits the K-extension operand of the big GEMM:
//               [hi(sU) | lo(sU)] in bf16.
//  colreduce  : part[c][col][j] = sum_{i in chunk c} G[i][col] V[i][j] on MFMA
//               (G^T as the row operand via 2-byte LDS gathers, V as bf16
//               hi + lo). G may be H = act(g) * u recomputed from g, u.
//  finish     : fixed-order sum over chunks, scale, bf16, any output stride.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace qlora {

// ------------------------------------------------------------------ rowdot --
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int RD_ROWS = 64, RD_KT = 128, RD_STAGES = 3;

// element offset of (row, 16-byte chunk) in a [rows][128] bf16 tile: 16
// chunks per 256-byte row, XOR-swizzled by row so the 16 lanes of a fragment
// read (16 rows, one chunk) hit 16 different bank groups.
__device__ __forceinline__ int rswz(int row, int chunk) { return row * RD_KT + ((chunk ^ (row & 15)) << 3); }

}  // namespace

int rowdot_splits(int M, int K) {
  const int blocks = (M + RD_ROWS - 1) / RD_ROWS;
  int ns = (1024 + blocks - 1) / blocks;
  const int kmax = (K + RD_KT - 1) / RD_KT;
  if (ns > kmax) ns = kmax;
  if (ns > 16) ns = 16;
  if (ns < 1) ns = 1;
  return ns;
}

// part[split][i][j] = sum over the split's K range of G[i][k] * L[j][k].
// 64 rows x 128 K per step, staged by direct-to-LDS loads in a 3-deep ring;
// wave w owns rows 16w..16w+15 and all RT*16 columns (MFMA 16x16x32).
// Several independent products with the same M and R run as one launch:
// blockIdx.z picks the job, and the grid's y extent covers the job with the
// most K splits.
template <int RT>
__global__ __launch_bounds__(256) void rowdot_kernel(RowJobs jobs, int M, int R) {
  constexpr int GB = RD_ROWS * RD_KT * 2;     // G tile bytes
  constexpr int LB = RT * 16 * RD_KT * 2;     // L tile bytes
  constexpr int STAGE = GB + LB;
  constexpr int NL = 4 + RT;                  // DMA instructions per stage per wave
  __shared__ __attribute__((aligned(1024))) uint8_t smem[RD_STAGES * STAGE];
  const int jb = blockIdx.z;
  if ((int)blockIdx.y >= jobs.nsplit[jb]) return;
  const uint16_t* __restrict__ G = jobs.G[jb];
  const int64_t ldg = jobs.ldg[jb];
  const uint16_t* __restrict__ L = jobs.L[jb];
  const int64_t ldl = jobs.ldl[jb];
  const int K = jobs.K[jb], kper = jobs.kper[jb];
  float* __restrict__ part = jobs.part[jb];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * RD_ROWS;
  const int kbeg = blockIdx.y * kper;
  const int kend = min(K, kbeg + kper);
  const int nst = (kend - kbeg + RD_KT - 1) / RD_KT;

  const uint16_t* srcG[4];
  int chG[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (wave * 4 + j) * 64 + lane;
    const int row = slot >> 4, chunk = (slot & 15) ^ (row & 15);
    srcG[j] = G + (int64_t)min(r0 + row, M - 1) * ldg;
    chG[j] = chunk * 8;
  }
  const uint16_t* srcL[RT];
  int chL[RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    const int slot = (wave * RT + j) * 64 + lane;
    const int row = slot >> 4, chunk = (slot & 15) ^ (row & 15);
    srcL[j] = L + (int64_t)min(row, R - 1) * ldl;
    chL[j] = chunk * 8;
  }

  auto issue = [&](int st) {
    uint8_t* b = smem + (st % RD_STAGES) * STAGE;
    const int k0 = kbeg + st * RD_KT;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = (k0 + chG[j] < kend) ? k0 + chG[j] : kbeg;  // past the end: any valid column
      dma16(srcG[j] + k, b + (wave * 4 + j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      const int k = (k0 + chL[j] < kend) ? k0 + chL[j] : kbeg;
      dma16(srcL[j] + k, b + GB + (wave * RT + j) * 1024);
    }
  };

  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int g = lane >> 4, m = lane & 15;

  const int npro = min(RD_STAGES - 1, nst);
  for (int st = 0; st < npro; ++st) issue(st);
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) wait_vm_lgkm0<NL>();   // this wave's stage st landed
    else wait_vm_lgkm0<0>();
    raw_barrier();
    if (st + RD_STAGES - 1 < nst) issue(st + RD_STAGES - 1);
    const uint16_t* sg = (const uint16_t*)(smem + (st % RD_STAGES) * STAGE);
    const uint16_t* sl = (const uint16_t*)(smem + (st % RD_STAGES) * STAGE + GB);
    const int nsub = min(RD_KT, kend - (kbeg + st * RD_KT)) >> 5;
    for (int ks = 0; ks < nsub; ++ks) {
      const bf16x8_t a = *(const bf16x8_t*)&sg[rswz(wave * 16 + m, 4 * ks + g)];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const bf16x8_t b = *(const bf16x8_t*)&sl[rswz(t * 16 + m, 4 * ks + g)];
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[t], 0, 0, 0);
      }
    }
  }
  // acc[t][v] = partial U[r0 + 16*wave + 4*g + v][t*16 + m]
  float* out = part + (int64_t)blockIdx.y * M * R;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = r0 + wave * 16 + 4 * g + v;
      const int j = t * 16 + m;
      if (row < M && j < R) out[(int64_t)row * R + j] = acc[t][v];
    }
}

// sum_{q < n} p[q * stride], added in order q = 0, 1, ... (the same bits as
// a plain loop); the loads are issued 8 at a time so that their latencies
// overlap instead of following one another.
__device__ __forceinline__ float ordered_sum(const float* __restrict__ p, int64_t stride, int n) {
  float sum = 0.0f;
  int q = 0;
  for (; q + 8 <= n; q += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(q + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  for (; q < n; ++q) sum += p[(int64_t)q * stride];
  return sum;
}

// The same sum for 4 consecutive columns (p 16-byte aligned, stride a
// multiple of 4): component-wise the same additions in the same order.
__device__ __forceinline__ f32x4_t ordered_sum4(const float* __restrict__ p, int64_t stride, int n) {
  f32x4_t sum = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  int q = 0;
  for (; q + 8 <= n; q += 8) {
    f32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const f32x4_t*)(p + (int64_t)(q + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  for (; q < n; ++q) sum += *(const f32x4_t*)(p + (int64_t)q * stride);
  return sum;
}

// U = sum of the split partials (fixed order); writes fp32 U (split across
// two outputs at column `split`) and the bf16 K-extension operand
// Ue = [hi(sU) | lo(sU) | 0]. A thread takes 4 consecutive columns of one row
// of [0, max(R, KE)): with R % 4 == 0 it reads them as one 16-byte partial.
// blockIdx.y picks the job; the grid covers the widest one
__global__ __launch_bounds__(256) void rowdot_finish_kernel(RowFinishJobs jobs, int M, int R,
                                                            float s) {
  const int jb = blockIdx.y;
  const float* __restrict__ part = jobs.part[jb];
  const int nsplit = jobs.nsplit[jb], split = jobs.split[jb], KE = jobs.KE[jb];
  float* __restrict__ Uf = jobs.Uf[jb];
  float* __restrict__ Uf2 = jobs.Uf2[jb];
  const int64_t ldu = jobs.ldu[jb], ldue = jobs.ldue[jb];
  uint16_t* __restrict__ Ue = jobs.Ue[jb];
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int W4 = ((KE > R ? KE : R) + 3) >> 2;
  if (e >= (int64_t)M * W4) return;
  const int i = (int)(e / W4), j0 = 4 * (int)(e - (int64_t)i * W4);
  float sum[4];
  if ((R & 3) == 0 && j0 < R) {
    const f32x4_t v = ordered_sum4(part + (int64_t)i * R + j0, (int64_t)M * R, nsplit);
#pragma unroll
    for (int t = 0; t < 4; ++t) sum[t] = v[t];
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      sum[t] = j0 + t < R ? ordered_sum(part + (int64_t)i * R + j0 + t, (int64_t)M * R, nsplit) : 0.0f;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = j0 + t;
    if (j < R) {
      if (j < split) {
        if (Uf) Uf[(int64_t)i * ldu + j] = sum[t];
      } else if (Uf2) {
        Uf2[(int64_t)i * ldu + (j - split)] = sum[t];
      }
      if (Ue) {
        const float su = s * sum[t];
        const uint32_t hi = f32_to_bf16(su);
        Ue[(int64_t)i * ldue + j] = (uint16_t)hi;
        Ue[(int64_t)i * ldue + R + j] = (uint16_t)f32_to_bf16(su - bf16_to_f32(hi));
      }
    } else if (Ue && j >= 2 * R && j < KE) {
      Ue[(int64_t)i * ldue + j] = 0;
    }
  }
}

hipError_t launch_rowdot_finish_jobs(const RowFinishJobs& jobs, int njobs, int M, int R, float s,
                                     hipStream_t stream) {
  if (M <= 0 || njobs <= 0) return hipSuccess;
  if (njobs > kMaxRowJobs || R < 1 || R > 64) return hipErrorInvalidValue;
  int64_t total = 0;
  for (int i = 0; i < njobs; ++i) {
    if (jobs.nsplit[i] < 1) return hipErrorInvalidValue;
    const int W4 = ((jobs.KE[i] > R ? jobs.KE[i] : R) + 3) / 4;
    total = std::max<int64_t>(total, (int64_t)M * W4);
  }
  rowdot_finish_kernel<<<dim3((unsigned)((total + 255) / 256), (unsigned)njobs), dim3(256), 0,
                         stream>>>(jobs, M, R, s);
  return hipGetLastError();
}

hipError_t launch_rowdot_jobs(const RowJobs& in, const RowFinishJobs& out, int njobs, int M, int R,
                              float s, hipStream_t stream) {
  if (M <= 0 || njobs <= 0) return hipSuccess;
  if (njobs > kMaxRowJobs || R < 1 || R > 64) return hipErrorInvalidValue;
  RowJobs jobs = in;
  RowFinishJobs fin = out;
  int nsmax = 1;
  for (int i = 0; i < njobs; ++i) {
    const int K = jobs.K[i];
    if (K <= 0 || K % 64) return hipErrorInvalidValue;
    const int ns = rowdot_splits(M, K);
    int kper = (K + ns - 1) / ns;
    kper = (kper + RD_KT - 1) / RD_KT * RD_KT;
    jobs.kper[i] = kper;
    jobs.nsplit[i] = (K + kper - 1) / kper;
    fin.part[i] = jobs.part[i];
    fin.nsplit[i] = jobs.nsplit[i];
    nsmax = std::max(nsmax, jobs.nsplit[i]);
  }
  dim3 grid((unsigned)((M + RD_ROWS - 1) / RD_ROWS), (unsigned)nsmax, (unsigned)njobs), block(256);
  switch ((R + 15) / 16) {
    case 1: rowdot_kernel<1><<<grid, block, 0, stream>>>(jobs, M, R); break;
    case 2: rowdot_kernel<2><<<grid, block, 0, stream>>>(jobs, M, R); break;
    case 3: rowdot_kernel<3><<<grid, block, 0, stream>>>(jobs, M, R); break;
    case 4: rowdot_kernel<4><<<grid, block, 0, stream>>>(jobs, M, R); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_rowdot_finish_jobs(fin, njobs, M, R, s, stream);
}

hipError_t launch_rowdot(const uint16_t* G, int64_t ldg, const uint16_t* L, int64_t ldl, int M,
                         int K, int R, float s, float* Uf, float* Uf2, int split, int64_t ldu,
                         uint16_t* Ue, int64_t ldue, int KE, float* part, hipStream_t stream) {
  RowJobs in{};
  RowFinishJobs out{};
  in.G[0] = G; in.ldg[0] = ldg; in.L[0] = L; in.ldl[0] = ldl; in.K[0] = K; in.part[0] = part;
  out.Uf[0] = Uf; out.Uf2[0] = Uf2; out.split[0] = split; out.ldu[0] = ldu; out.Ue[0] = Ue;
  out.ldue[0] = ldue; out.KE[0] = KE;
  return launch_rowdot_jobs(in, out, 1, M, R, s, stream);
}

hipError_t launch_rowdot_finish(const float* part, int nsplit, int M, int R, float s, float* Uf,
                                float* Uf2, int split, int64_t ldu, uint16_t* Ue, int64_t ldue,
                                int KE, hipStream_t stream) {
  RowFinishJobs out{};
  out.part[0] = part; out.nsplit[0] = nsplit; out.Uf[0] = Uf; out.Uf2[0] = Uf2;
  out.split[0] = split; out.ldu[0] = ldu; out.Ue[0] = Ue; out.ldue[0] = ldue; out.KE[0] = KE;
  return launch_rowdot_finish_jobs(out, 1, M, R, s, stream);
}

// --------------------------------------------------------------- colreduce --
int colreduce_chunks(int M) {
  int c = (M + 255) / 256;
  if (c < 1) c = 1;
  if (c > 32) c = 32;
  return c;
}

// part[chunk][col][j] = sum over the chunk's rows i of G[i][col] * V[i][j].
// MFMA 16x16x32 with D[col][j] = sum_k G^T[col][k] V[k][j]: a block owns 256
// columns and walks its rows 32 at a time. The 32 x 256 G tile is staged in
// LDS with a 544-byte row pitch; lane group g = lane/16 takes rows 4t + g
// (t = 0..7) of the step as its 8 K-elements (a fixed permutation of K, used
// for both operands), so each 2-byte gather of a fragment hits 4 distinct
// 32-byte bank groups. V is split into bf16 hi + lo (V - hi) halves, stored
// transposed and permuted, so its fragments are single 16-byte LDS reads;
// hi and lo are accumulated by two MFMAs into the same fp32 sum.
// HMODE: G = H = bf16(act(g) * u), recomputed from g and u.
// Several independent reductions of one shape class (same M, R, ldv) run as
// one launch: blockIdx.z picks the job.
template <int RT, bool HMODE>
__global__ __launch_bounds__(256) void colreduce_kernel(ColJobs jobs,
                                                        const uint16_t* __restrict__ gate,
                                                        const uint16_t* __restrict__ up, int act,
                                                        int M, int64_t ldv, int R,
                                                        int rows_per_chunk) {
  constexpr int CT = 256, KS = 32, PITCH = 544;
  __shared__ __attribute__((aligned(16))) uint8_t gt[2][KS * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][2][RT * 16][KS];
  const int jb = blockIdx.z;
  const uint16_t* __restrict__ G = jobs.G[jb];
  const int64_t ldg = jobs.ldg[jb];
  const int C = jobs.C[jb];
  const float* __restrict__ V = jobs.V[jb];
  float* __restrict__ part = jobs.part[jb];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * CT;
  if (c0 >= C) return;   // the grid covers the widest job
  const int chunk = blockIdx.y;
  const int r0 = chunk * rows_per_chunk;
  const int r1 = min(M, r0 + rows_per_chunk);
  const int nsteps = (r1 - r0 + KS - 1) / KS;

  // padding columns j >= R of the V tiles stay zero
  for (int e = tid; e < 2 * 2 * RT * 16 * KS; e += 256) (&vt[0][0][0][0])[e] = 0;

  // G tile loads: 32 rows x 32 chunks of 16 B; thread t takes chunks t + 256 q
  constexpr int NV = 2 * RT;  // V values per thread per step (32 rows x RT*16 cols)
  u32x4_t rg[4];
  u32x4_t ru[HMODE ? 4 : 1];
  float rv[NV];
  auto load = [&](int st) {
    const int rbase = r0 + st * KS;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q;
      const int row = min(rbase + (idx >> 5), M - 1);
      const int col = min(c0 + (idx & 31) * 8, C - 8);
      if (HMODE) {
        rg[q] = *(const u32x4_t*)(gate + (int64_t)row * ldg + col);
        ru[q] = *(const u32x4_t*)(up + (int64_t)row * ldg + col);
      } else {
        rg[q] = *(const u32x4_t*)(G + (int64_t)row * ldg + col);
      }
    }
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int idx = tid + 256 * q;
      const int row = rbase + idx / R;
      rv[q] = (idx < KS * R && row < r1) ? V[(int64_t)row * ldv + idx % R] : 0.0f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q;
      u32x4_t v = rg[q];
      if (HMODE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float h0 = act_fwd(act, bf16_to_f32(rg[q][e] & 0xFFFFu)) * bf16_to_f32(ru[q][e] & 0xFFFFu);
          const float h1 = act_fwd(act, bf16_to_f32(rg[q][e] >> 16)) * bf16_to_f32(ru[q][e] >> 16);
          v[e] = pack_bf16x2(h0, h1);
        }
      }
      *(u32x4_t*)&gt[buf][(idx >> 5) * PITCH + (idx & 31) * 16] = v;
    }
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int idx = tid + 256 * q;
      if (idx < KS * R) {
        const int row = idx / R, j = idx % R;
        const int pp = 8 * (row & 3) + (row >> 2);
        const uint32_t hi = f32_to_bf16(rv[q]);
        vt[buf][0][j][pp] = (uint16_t)hi;
        vt[buf][1][j][pp] = (uint16_t)f32_to_bf16(rv[q] - bf16_to_f32(hi));
      }
    }
  };

  f32x4_t acc[4][RT];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) acc[ct][jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int g = lane >> 4, m = lane & 15;
  if (nsteps > 0) {
    load(0);
    __syncthreads();  // zero-fill of vt done before the first store
    store(0);
    __syncthreads();
  }
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (st + 1 < nsteps) load(st + 1);
    bf16x8_t bh[RT], bl[RT];
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) {
      bh[jt] = *(const bf16x8_t*)&vt[buf][0][jt * 16 + m][8 * g];
      bl[jt] = *(const bf16x8_t*)&vt[buf][1][jt * 16 + m][8 * g];
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const uint8_t* base = &gt[buf][(wave * 64 + ct * 16 + m) * 2];
      bf16x8_t a;
#pragma unroll
      for (int t = 0; t < 8; ++t) a[t] = *(const __bf16*)(base + (4 * t + g) * PITCH);
#pragma unroll
      for (int jt = 0; jt < RT; ++jt) {
        acc[ct][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[jt], acc[ct][jt], 0, 0, 0);
        acc[ct][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[jt], acc[ct][jt], 0, 0, 0);
      }
    }
    if (st + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }
  // acc[ct][jt][v] = part for column c0 + wave*64 + ct*16 + 4*g + v, j = jt*16 + m
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int jt = 0; jt < RT; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int col = c0 + wave * 64 + ct * 16 + 4 * g + v;
        const int j = jt * 16 + m;
        if (col < C && j < R) part[((int64_t)chunk * C + col) * R + j] = acc[ct][jt][v];
      }
}

hipError_t launch_colreduce_jobs(const ColJobs& jobs, int njobs, const uint16_t* gate,
                                 const uint16_t* up, int act, int M, int64_t ldv, int R,
                                 hipStream_t stream) {
  if (M <= 0 || njobs <= 0) return hipSuccess;
  if (njobs > kMaxColJobs || R < 1 || R > 64) return hipErrorInvalidValue;
  int cmax = 0;
  for (int i = 0; i < njobs; ++i) {
    if (jobs.C[i] <= 0 || jobs.C[i] % 8) return hipErrorInvalidValue;
    cmax = std::max(cmax, jobs.C[i]);
  }
  const int chunks = colreduce_chunks(M);
  const int rpc = (M + chunks - 1) / chunks;
  dim3 grid((unsigned)((cmax + 255) / 256), (unsigned)chunks, (unsigned)njobs), block(256);
  const bool hm = gate != nullptr;
#define QL_CR(RTV)                                                                              \
  do {                                                                                          \
    if (hm)                                                                                     \
      colreduce_kernel<RTV, true><<<grid, block, 0, stream>>>(jobs, gate, up, act, M, ldv, R,   \
                                                              rpc);                             \
    else                                                                                        \
      colreduce_kernel<RTV, false><<<grid, block, 0, stream>>>(jobs, gate, up, act, M, ldv, R,  \
                                                               rpc);                            \
  } while (0)
  if (R <= 16) QL_CR(1);
  else if (R <= 32) QL_CR(2);
  else QL_CR(4);
#undef QL_CR
  return hipGetLastError();
}

hipError_t launch_colreduce(const uint16_t* G, const uint16_t* gate, const uint16_t* up, int act,
                            int64_t ldg, int M, int C, const float* V, int64_t ldv, int R,
                            float* part, hipStream_t stream) {
  if (M <= 0 || C <= 0) return hipSuccess;
  ColJobs j{};
  j.G[0] = G; j.ldg[0] = ldg; j.C[0] = C; j.V[0] = V; j.part[0] = part;
  return launch_colreduce_jobs(j, 1, gate, up, act, M, ldv, R, stream);
}

// blockIdx.y picks the job; the grid covers the largest one
__global__ __launch_bounds__(256) void colreduce_finish_kernel(ColFinishJobs jobs, int chunks,
                                                               int nj, float s) {
  const int jb = blockIdx.y;
  const float* __restrict__ part = jobs.part[jb];
  const int C = jobs.C[jb], R = jobs.R[jb], j0 = jobs.j0[jb];
  uint16_t* __restrict__ out = jobs.out[jb];
  const int64_t ocs = jobs.ocs[jb], ojs = jobs.ojs[jb];
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)C * nj) return;
  const int col = (int)(e / nj);
  const int jj = (int)(e - (int64_t)col * nj);
  const float sum = ordered_sum(part + (int64_t)col * R + j0 + jj, (int64_t)C * R, chunks);
  out[(int64_t)col * ocs + (int64_t)jj * ojs] = (uint16_t)f32_to_bf16(s * sum);
}

hipError_t launch_colreduce_finish_jobs(const ColFinishJobs& jobs, int njobs, int chunks, int nj,
                                        float s, hipStream_t stream) {
  if (njobs <= 0 || nj <= 0) return hipSuccess;
  if (njobs > kMaxColJobs) return hipErrorInvalidValue;
  int64_t total = 0;
  for (int i = 0; i < njobs; ++i) total = std::max<int64_t>(total, (int64_t)jobs.C[i] * nj);
  if (total <= 0) return hipSuccess;
  colreduce_finish_kernel<<<dim3((unsigned)((total + 255) / 256), (unsigned)njobs), dim3(256), 0,
                            stream>>>(jobs, chunks, nj, s);
  return hipGetLastError();
}

hipError_t launch_colreduce_finish(const float* part, int chunks, int C, int R, int j0, int nj,
                                   float s, uint16_t* out, int64_t ocs, int64_t ojs,
                                   hipStream_t stream) {
  ColFinishJobs j{};
  j.part[0] = part; j.C[0] = C; j.R[0] = R; j.j0[0] = j0; j.out[0] = out; j.ocs[0] = ocs; j.ojs[0] = ojs;
  return launch_colreduce_finish_jobs(j, 1, chunks, nj, s, stream);
}

// ---------------------------------------------------------------- layout --
// All small LoRA operand layouts of one entry point in a single launch: job j
// (blockIdx.y) copies a strided rows x cols view (or writes zeros when its
// source is null). Jobs never overlap, so their order does not matter.
// A thread takes up to 8 elements, spaced by the grid's thread count, and
// loads all of its batch before it stores any of it (sources and
// destinations of the jobs are disjoint). Few workgroups per job: when this
// launch runs beside another kernel, its workgroups are dispatched in turn
// with that kernel's, so a wide grid had stretched it several-fold.
__global__ __launch_bounds__(256) void prep_kernel(PrepJobs jobs) {
  constexpr int U = 8;
  const PrepJob& jb = jobs.j[blockIdx.y];
  const int64_t total = (int64_t)jb.rows * jb.cols;
  if (total <= 0) return;
  const int64_t stride = (int64_t)gridDim.x * 256;
  // element e (clamped to the job, so that every load is in bounds and none
  // sits behind a branch): its destination and source offsets
  // (job sizes fit 32 bits, which keeps the division short; the host checks)
  auto offs = [&](int64_t e, int64_t& d, int64_t& sidx) {
    const int r = (int)((uint32_t)e / (uint32_t)jb.cols);
    const int c = (int)e - r * jb.cols;
    int64_t dr = r;
    if (jb.interleave) dr = 64 * (r >> 5) + 32 * (jb.interleave - 1) + (r & 31);
    d = dr * jb.d_rs + (int64_t)c * jb.d_cs;
    sidx = (int64_t)r * jb.s_rs + (int64_t)c * jb.s_cs;
  };
  for (int64_t e0 = (int64_t)blockIdx.x * 256 + threadIdx.x; e0 < total; e0 += U * stride) {
    uint16_t v[U];
    int64_t d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t sidx;
      offs(min(e0 + u * stride, total - 1), d[u], sidx);
      v[u] = jb.src ? jb.src[sidx] : (uint16_t)0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (e0 + u * stride < total) jb.dst[d[u]] = v[u];
  }
}

hipError_t launch_prep(const PrepJobs& jobs, hipStream_t stream) {
  if (jobs.n <= 0) return hipSuccess;
  if (jobs.n > kMaxPrepJobs) return hipErrorInvalidValue;
  int64_t most = 0;
  for (int i = 0; i < jobs.n; ++i) {
    const int64_t t = (int64_t)jobs.j[i].rows * jobs.j[i].cols;
    if (jobs.j[i].rows < 0 || jobs.j[i].cols < 0 || t >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    most = std::max(most, t);
  }
  int64_t bx = (most + 256 * 8 - 1) / (256 * 8);   // one batch of 8 per thread
  if (bx < 1) bx = 1;
  if (bx > 64) bx = 64;
  prep_kernel<<<dim3((unsigned)bx, (unsigned)jobs.n), dim3(256), 0, stream>>>(jobs);
  return hipGetLastError();
}

// Zero-fill by a kernel (not hipMemsetAsync) so callers may capture the
// sequence in a graph.
__global__ __launch_bounds__(256) void zero_kernel(uint8_t* __restrict__ dst, size_t bytes) {
  const size_t n16 = bytes >> 4;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    ((u32x4_t*)dst)[i] = u32x4_t{0u, 0u, 0u, 0u};
  const size_t tail = bytes & 15;
  if (blockIdx.x == 0 && threadIdx.x < tail) dst[(n16 << 4) + threadIdx.x] = 0;
}

hipError_t launch_zero(void* dst, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = ((bytes >> 4) + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>((uint8_t*)dst, bytes);
  return hipGetLastError();
}

}  // namespace qlora
