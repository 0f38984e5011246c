// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

void nf4_levels_host(float out[16]);

// fp32 absmax of an NF4 weight [n][k/64] (flattened index i = row * k/64 +
// block), stored as it is (f32) or double-quantized: 8-bit codes q with one
// fp32 scale and offset per 256 consecutive values,
//   absmax[i] = fp32(fp32(q[i] * scale[i / 256]) + offset[i / 256]).
struct AbsmaxSrc {
  const float* f32;      // plain fp32 array, or null when double-quantized
  const int8_t* q;
  const float* scale;
  const float* offset;
};
constexpr int kDqGroup = 256;

// ---- NF4 dequant (nf4.hip) ----
// out[dest_row(i)][j] = W[i][j]; interleave 0: dest_row(i) = i; 1/2: the 32-row
// interleave of a gate (1) / up (2) pair: 64*(i/32) + 32*(interleave-1) + i%32.
hipError_t launch_nf4_dequant_rows(const uint8_t* codes, AbsmaxSrc absmax, int64_t n, int64_t k,
                                   uint16_t* out, int64_t ld_out, int interleave,
                                   hipStream_t stream);
// out[j][col_ofs + i] = W[i][j]   (n, k multiples of 64)
hipError_t launch_nf4_dequant_transpose(const uint8_t* codes, AbsmaxSrc absmax, int64_t n,
                                        int64_t k, uint16_t* out, int64_t ld_out, int64_t col_ofs,
                                        hipStream_t stream);

// Double quantization of an fp32 absmax array of nb values (groups of 256):
// offset = fp32(sequential fp64 sum / count), scale = fp32(max |a - offset| /
// 127) in fp64, q = clamp(rne((a - offset) / scale), -127, 127) (0 if scale is 0).
hipError_t launch_absmax_dq_quantize(const float* absmax, int64_t nb, int8_t* q, float* scale,
                                     float* offset, hipStream_t stream);
// out[i] = the reconstructed absmax (fp32), i < nb
hipError_t launch_absmax_dq_dequant(const int8_t* q, const float* scale, const float* offset,
                                    int64_t nb, float* out, hipStream_t stream);

// NF4 quantizer: codes [n][k/2] and absmax [n][k/64] from bf16 W [n][k]
hipError_t launch_nf4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                               float* absmax, hipStream_t stream);

// ---- bf16 base-weight staging (w16.hip); n, k multiples of 64 ----
// out[dest_row(i)][j] = W[i][j] (dest_row as for the NF4 dequant)
hipError_t launch_w16_rows(const uint16_t* src, int64_t n, int64_t k, uint16_t* out, int64_t ld_out,
                           int interleave, hipStream_t stream);
// out[j][col_ofs + i] = W[i][j]
hipError_t launch_w16_transpose(const uint16_t* src, int64_t n, int64_t k, uint16_t* out,
                                int64_t ld_out, int64_t col_ofs, hipStream_t stream);

// ---- GEMM (gemm.hip) ----
enum GemmEpilogue {
  EPI_STORE = 0,     // C bf16 [M][N]
  EPI_GATEUP = 1,    // columns interleaved by 32 (gate, up); writes g, u, H = act(g) * u
  EPI_ACT_BWD = 2,   // C = dH [M][h]; reads g, u; writes dgu = [dg | du] [M][2h]
  EPI_STORE3 = 3,    // bf16 columns [0, nc1) to C, [nc1, nc2) to C1, [nc2, N) to C2
                     // (bf16 B source only; nc1, nc2 multiples of 8)
};

// How the B operand ([N][K] weight, K contiguous) reaches the tile:
//   bf16 rows, or NF4 codes dequantized while the tile is staged in LDS.
enum GemmBSource {
  BSRC_BF16 = 0,      // B bf16 [N][K]
  BSRC_NF4 = 1,       // B = NF4 weight [N][K]
  BSRC_NF4_PAIR = 2,  // B rows interleaved by 32 from two NF4 weights [N/2][K] (gate, up)
  BSRC_NF4_T = 3      // B = W^T for an NF4 weight W [K][N]; with codes1, W = [W0; W1]
                      // stacked along K (rows >= ksplit come from W1)
};

struct GemmArgs {
  // main operands: A [M][K] bf16 (lda); B [N][K] bf16 (ldb) or NF4
  const uint16_t* A;
  int64_t lda;
  // bf16 B source only: A split along K into segments, K columns [0, ka1) from
  // A, [ka1, ka2) from A1 (lda1), [ka2, K) from A2 (lda2); ka1 <= ka2 <= K,
  // multiples of 64. A1 == nullptr: one segment.
  const uint16_t* A1;
  int64_t lda1;
  const uint16_t* A2;
  int64_t lda2;
  int ka1, ka2;
  const uint16_t* B;
  int64_t ldb;
  int bsrc;
  const uint8_t* codes0;   // NF4 of B rows (pair mode: gate rows)
  const float* absmax0;
  const uint8_t* codes1;   // pair mode: up rows; transposed mode: second stacked weight
  const float* absmax1;
  int ksplit;              // transposed mode: first K index served by codes1 (0 = none)
  // K-extension: C += Ae [M][KE] * Be [N][KE]^T (KE multiple of 16, may be 0)
  const uint16_t* Ae;
  int64_t ldae;
  const uint16_t* Be;
  int64_t ldbe;
  int M, N, K, KE;
  // split-K (EPI_STORE / EPI_STORE3): splits > 1 runs each
  // tile as `splits` K ranges writing fp32 partials part [splits][M][N], then a
  // reduction sums them in order and stores; the K-extension rides on split 0
  int splits;
  float* part;
  // epilogue
  int epi;
  uint16_t* C;
  int64_t ldc;
  uint16_t* C1;   // EPI_STORE3
  int64_t ldc1;
  uint16_t* C2;
  int64_t ldc2;
  int nc1, nc2;
  uint16_t* g_out;
  uint16_t* u_out;
  uint16_t* h_out;
  const uint16_t* g_in;
  const uint16_t* u_in;
  uint16_t* dgu;
  int64_t hdim;
  int act;
  // row product in the GATEUP / ACT_BWD epilogues (gemm_bf16_kernel only):
  // with rp_r in 1..16, the bf16 values the epilogue writes (H; dg and du)
  // are multiplied by a rank-r operand over the tile's columns into an fp32
  // partial part[tile_col][row][j]; gemm_rowprod_splits(N) partials per row,
  // summed by launch_rowdot_finish.
  //   GATEUP:  j < r: sum_c H[row][c] rp_l[j][c]                  (width r)
  //   ACT_BWD: j < r: sum_c dg[row][c] rp_l[j][c]; r + j: sum_c du[row][c]
  //            rp_l2[j][c]                                        (width 2r)
  // rp_l, rp_l2: bf16 with row pitch rp_ldl; c runs over [0, hdim).
  const uint16_t* rp_l;
  const uint16_t* rp_l2;
  int64_t rp_ldl;
  int rp_r;   // 0: off
  float* rp_part;
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
// K splits for an M x N x K product with a store epilogue: enough to give
// about 256 concurrent tiles when the output has fewer, each split at least 8
// k-steps of 64, at most 8 splits, every split non-empty. A fixed function of
// the shape, so workspace queries and launches agree.
int gemm_splits(int M, int N, int K);
// partials per row written by the epilogue row product of an N-column GEMM
int gemm_rowprod_splits(int N);

// ---- LoRA skinny kernels (lora.hip) ----
// U = G L^T for G [M][K] bf16 (ldg), L [R][K] bf16 (ldl), 1 <= R <= 64.
// Writes columns j < split to Uf [M][ldu] and j >= split to Uf2 (column
// j - split) as fp32 (either may be null) and, if Ue is non-null,
// Ue [M][KE] bf16 = [hi(s U) | lo(s U) | 0 ...] with hi = bf16(sU),
// lo = bf16(sU - hi), KE = ceil16(2R).
// part: scratch of rowdot_splits(M, K) * M * R floats.
int rowdot_splits(int M, int K);
hipError_t launch_rowdot(const uint16_t* G, int64_t ldg, const uint16_t* L, int64_t ldl, int M,
                         int K, int R, float s, float* Uf, float* Uf2, int split, int64_t ldu,
                         uint16_t* Ue, int64_t ldue, int KE, float* part, hipStream_t stream);
// The fixed-order sum of nsplit partials part [nsplit][M][R] and the outputs
// of launch_rowdot (Uf, Uf2, Ue) from it.
hipError_t launch_rowdot_finish(const float* part, int nsplit, int M, int R, float s, float* Uf,
                                float* Uf2, int split, int64_t ldu, uint16_t* Ue, int64_t ldue,
                                int KE, hipStream_t stream);
// Up to kMaxRowJobs independent products with the same M and R in one launch
// per stage: job i is what launch_rowdot(in.G[i], in.ldg[i], in.L[i],
// in.ldl[i], M, in.K[i], R, s, out.Uf[i], out.Uf2[i], out.split[i],
// out.ldu[i], out.Ue[i], out.ldue[i], out.KE[i], in.part[i]) computes, with
// its own partial buffer (the split counts and K ranges are filled in here).
constexpr int kMaxRowJobs = 3;
struct RowJobs {
  const uint16_t* G[kMaxRowJobs];
  int64_t ldg[kMaxRowJobs];
  const uint16_t* L[kMaxRowJobs];
  int64_t ldl[kMaxRowJobs];
  int K[kMaxRowJobs];
  int kper[kMaxRowJobs];
  int nsplit[kMaxRowJobs];
  float* part[kMaxRowJobs];
};
struct RowFinishJobs {
  const float* part[kMaxRowJobs];
  int nsplit[kMaxRowJobs];
  float* Uf[kMaxRowJobs];
  float* Uf2[kMaxRowJobs];
  int split[kMaxRowJobs];
  int64_t ldu[kMaxRowJobs];
  uint16_t* Ue[kMaxRowJobs];
  int64_t ldue[kMaxRowJobs];
  int KE[kMaxRowJobs];
};
hipError_t launch_rowdot_jobs(const RowJobs& in, const RowFinishJobs& out, int njobs, int M, int R,
                              float s, hipStream_t stream);
hipError_t launch_rowdot_finish_jobs(const RowFinishJobs& jobs, int njobs, int M, int R, float s,
                                     hipStream_t stream);

// Column reduction over tokens, first stage: for each chunk c of rows,
// part[c][col][j] = sum_{i in chunk} G[i][col] * V[i][vofs + j], j < R.
// G is bf16 [M][C] (ldg) or, when gate/up are given, H = act(g) * u
// recomputed from bf16 g, u [M][C] (ldg).
int colreduce_chunks(int M);
hipError_t launch_colreduce(const uint16_t* G, const uint16_t* gate, const uint16_t* up, int act,
                            int64_t ldg, int M, int C, const float* V, int64_t ldv, int R,
                            float* part, hipStream_t stream);
// Second stage: out[col * ocs + (j - j0) * ojs] = bf16(s * sum_c part[c][col][j]), j0 <= j < j0+nj.
hipError_t launch_colreduce_finish(const float* part, int chunks, int C, int R, int j0, int nj,
                                   float s, uint16_t* out, int64_t ocs, int64_t ojs,
                                   hipStream_t stream);
// Up to kMaxColJobs independent reductions in one launch each: the first
// stage for jobs that share M, R and ldv (each with its own G, ldg, C, V and
// partial buffer), the second for jobs that share chunks, nj and s. Each job
// computes exactly what the single-job call computes.
constexpr int kMaxColJobs = 3;
struct ColJobs {
  const uint16_t* G[kMaxColJobs];
  int64_t ldg[kMaxColJobs];
  int C[kMaxColJobs];
  const float* V[kMaxColJobs];
  float* part[kMaxColJobs];
};
struct ColFinishJobs {
  const float* part[kMaxColJobs];
  int C[kMaxColJobs];
  int R[kMaxColJobs];
  int j0[kMaxColJobs];
  uint16_t* out[kMaxColJobs];
  int64_t ocs[kMaxColJobs];
  int64_t ojs[kMaxColJobs];
};
hipError_t launch_colreduce_jobs(const ColJobs& jobs, int njobs, const uint16_t* gate,
                                 const uint16_t* up, int act, int M, int64_t ldv, int R,
                                 hipStream_t stream);
hipError_t launch_colreduce_finish_jobs(const ColFinishJobs& jobs, int njobs, int chunks, int nj,
                                        float s, hipStream_t stream);

// ---- small layout kernels (lora.hip) ----
// One copy (src != null) or zero-fill (src == null) job:
// dst[drow(r) * d_rs + c * d_cs] = src[r * s_rs + c * s_cs] for r < rows, c < cols;
// drow(r) = r, or the 32-row interleave (as for the dequant) when interleave > 0.
struct PrepJob {
  const uint16_t* src;
  int64_t s_rs, s_cs;
  int rows, cols;
  uint16_t* dst;
  int64_t d_rs, d_cs;
  int interleave;
};
constexpr int kMaxPrepJobs = 24;
struct PrepJobs {
  PrepJob j[kMaxPrepJobs];
  int n = 0;
  // a job past the capacity is not stored; n then exceeds it and launch_prep
  // reports the overflow
  void copy(const uint16_t* src, int64_t s_rs, int64_t s_cs, int64_t rows, int64_t cols,
            uint16_t* dst, int64_t d_rs, int64_t d_cs, int interleave = 0) {
    if (n < kMaxPrepJobs)
      j[n] = PrepJob{src, s_rs, s_cs, (int)rows, (int)cols, dst, d_rs, d_cs, interleave};
    ++n;
  }
  void zero(int64_t rows, int64_t cols, uint16_t* dst, int64_t d_rs, int64_t d_cs,
            int interleave = 0) {
    if (rows > 0 && cols > 0) copy(nullptr, 0, 0, rows, cols, dst, d_rs, d_cs, interleave);
  }
};
// Jobs must write disjoint elements (they run concurrently).
hipError_t launch_prep(const PrepJobs& jobs, hipStream_t stream);
hipError_t launch_zero(void* dst, size_t bytes, hipStream_t stream);

// ---- RMS layernorm, RoPE, cross entropy (fast.hip) ----
// rmsnorm: X, Y, dY, dX [m][d] bf16 (d % 8 == 0), w [d] bf16; gemma: scale
// by 1 + w instead of w; rstd [m] fp32 = 1/rms (forward output, backward input)
hipError_t launch_rmsnorm_fwd(const uint16_t* X, int64_t m, int64_t d, const uint16_t* w, float eps,
                              int gemma, uint16_t* Y, float* rstd, hipStream_t stream);
hipError_t launch_rmsnorm_bwd(const uint16_t* dY, const uint16_t* X, const float* rstd, int64_t m,
                              int64_t d, const uint16_t* w, int gemma, uint16_t* dX,
                              hipStream_t stream);
// RoPE on X [m][heads][hd] (row pitch ldx), half-split pairs (j, j + hd/2);
// inv_freq[j] = base^(-2j/hd) in fp64 (hd % 16 == 0, hd <= 256); backward
// rotates by the opposite angle. Y may be X (same pitch).
struct RopeFreq {
  double inv_freq[128];
};
hipError_t launch_rope(const uint16_t* X, int64_t ldx, uint16_t* Y, int64_t ldy, int64_t m, int heads,
                       int hd, const int64_t* pos, const RopeFreq& fr, int backward,
                       hipStream_t stream);
// cross entropy over logits X [m][V] (row pitch ld, a multiple of 8); labels
// int64 [m] (outside [0, V): no target). Forward: lse, ce [m] fp32, loss and
// n_valid (device scalars). Backward: dX [m][V] (pitch ldd), may be X.
hipError_t launch_xent_fwd(const uint16_t* X, int64_t ld, int64_t m, int64_t V, const int64_t* labels,
                           float* lse, float* ce, float* loss, int32_t* n_valid, hipStream_t stream);
// forward and backward in one visit of each row; dloss is the upstream scale
hipError_t launch_xent_fused(const uint16_t* X, int64_t ld, int64_t m, int64_t V, const int64_t* labels,
                             float dloss, float* lse, float* ce, float* loss, int32_t* n_valid,
                             uint16_t* dX, int64_t ldd, hipStream_t stream);
hipError_t launch_xent_bwd(const uint16_t* X, int64_t ld, int64_t m, int64_t V, const int64_t* labels,
                           const float* lse, const float* dloss, const int32_t* n_valid, uint16_t* dX,
                           int64_t ldd, hipStream_t stream);

// ---- scratch of the no-allocation entry point (scratch.hip) ----
// A file-scope device array of kScratchBytes per GPU, held from module load
// until the process ends; scratch_device_ptr gives the current device's copy
// (looked up once per device). Calls that use it must not overlap on a GPU.
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_device_ptr(void** out);

// ---- diagnostics (probe.hip) ----
// Sustained dense bf16 MFMA TFLOP/s and the shader clock (GHz) under that
// load; synchronizes the host.
hipError_t probe_mfma_peak(int iters, hipStream_t stream, double* tflops, double* ghz);

}  // namespace qlora
