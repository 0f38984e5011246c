// bf16 MFMA GEMM for gfx950: C[M][N] = A[M][K] B[N][K]^T (+ Ae Be^T), fp32 accumulate.
//
// This is the dense contraction of every base projection of the QLoRA layer
// (the pages' profiling remark: runtime is dominated by the large MLP
// matmuls; Show HN thread) with the rank-r LoRA product folded in as a
// K-extension: for Y = X W^T + s (X A^T) B^T the caller passes
// Ae = [hi(sU) | lo(sU)] and Be = [B | B] (U = X A^T formed first, so the
// merged weight W + s B A never exists; Mistral benchmark page, items 10-11).
// hi/lo is a two-term bf16 split of the fp32 product, which keeps the LoRA
// term accurate to ~2^-17 relative on bf16 matrix cores.
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2), each wave
// 128 x 128 = 4 x 4 MFMA 32x32x16 tiles (256 fp32 accumulators per lane in
// AGPR/VGPR). K is walked in 64-wide steps through two LDS stages (2 x 64 KB
// of the 160 KB per CU): global loads of step k+1 are in flight while the
// matrix cores work on step k. LDS rows are 128 B with the 16-byte chunk index
// XOR-swizzled by (row & 7), so both the row-contiguous stores and the
// MFMA fragment reads (lane -> row lane%32, chunk 2ks + lane/32) are
// bank-conflict free.
//
// Weight operand B comes either as bf16 rows or as NF4 codes that are
// dequantized while the tile is staged into LDS (one weight row per thread,
// 64 weights = exactly one absmax block per K-step).
//
// Tile order: workgroup ids are dealt to the 8 XCDs round-robin; ids are
// remapped so that each XCD walks a contiguous range of tiles, grouped 8
// M-tiles at a time, which keeps shared A rows / B columns in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"
#include "nf4_table.hpp"

namespace qlora {

namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;

// element offset of (row, 16-byte chunk) in a [rows][64] bf16 LDS tile
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

__device__ __forceinline__ int xcd_remap(int pid, int n) {
  const int X = 8;
  int q = n / X, rmd = n % X;
  int xcd = pid % X, local = pid / X;
  return (xcd < rmd ? xcd * (q + 1) : rmd * (q + 1) + (xcd - rmd) * q) + local;
}

__device__ __forceinline__ u32x4_t dq8(uint32_t word, float amax, const float* lut) {
  u32x4_t o;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t byte = (word >> (8 * b)) & 0xFFu;
    float w0 = lut[byte >> 4] * amax;
    float w1 = lut[byte & 0xFu] * amax;
    o[b] = pack_bf16x2(w0, w1);
  }
  return o;
}

}  // namespace

__constant__ uint32_t c_nf4_levels_gemm[16] = {QLORA_NF4_LEVEL_BITS};

template <int BSRC, int EPI>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_nt_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * BK];
  __shared__ float lut[16];
  uint16_t (*sA)[BM * BK] = reinterpret_cast<uint16_t (*)[BM * BK]>(smem);
  uint16_t (*sB)[BN * BK] = reinterpret_cast<uint16_t (*)[BN * BK]>(smem + 2 * BM * BK);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  if (BSRC != BSRC_BF16) {
    if (tid < 16) lut[tid] = __uint_as_float(c_nf4_levels_gemm[tid]);
  }

  const int ntm = (p.M + BM - 1) / BM, ntn = (p.N + BN - 1) / BN;
  const int pid = xcd_remap(blockIdx.x, ntm * ntn);
  const int GM = 8;
  const int per_group = GM * ntn;
  const int group = pid / per_group;
  const int first_m = group * GM;
  const int gsz = min(ntm - first_m, GM);
  const int tm = first_m + (pid % per_group) % gsz;
  const int tn = (pid % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int nk_main = p.K / BK;
  const int nk_ext = (p.KE + BK - 1) / BK;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // ---- staging registers ----
  u32x4_t ra[8];
  u32x4_t rb[8];
  u32x4_t rc[2];
  float ramax = 0.0f;

  const int ld_row = tid >> 3, ld_chunk = tid & 7;

  // B-row source of tile row t (NF4 modes): plain or the 32-row gate/up interleave
  const uint8_t* nf_codes = p.codes0;
  const float* nf_amax = p.absmax0;
  int64_t nf_row = 0;
  if (BSRC != BSRC_BF16) {
    int gn = min(n0 + tid, p.N - 1);
    if (BSRC == BSRC_NF4_PAIR) {
      int which = (gn >> 5) & 1;
      nf_row = (int64_t)((gn >> 6) << 5) + (gn & 31);
      nf_codes = which ? p.codes1 : p.codes0;
      nf_amax = which ? p.absmax1 : p.absmax0;
    } else {
      nf_row = gn;
    }
  }

  auto load_main = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int gr = min(m0 + ld_row + 32 * i, p.M - 1);
      ra[i] = *(const u32x4_t*)(p.A + (int64_t)gr * p.lda + k0 + ld_chunk * 8);
    }
    if (BSRC == BSRC_BF16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int gr = min(n0 + ld_row + 32 * i, p.N - 1);
        rb[i] = *(const u32x4_t*)(p.B + (int64_t)gr * p.ldb + k0 + ld_chunk * 8);
      }
    } else {
      const uint8_t* src = nf_codes + nf_row * (int64_t)(p.K >> 1) + (k0 >> 1);
      rc[0] = *(const u32x4_t*)src;
      rc[1] = *(const u32x4_t*)(src + 16);
      ramax = nf_amax[nf_row * (int64_t)(p.K >> 6) + kt];
    }
  };

  auto store_main = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4_t*)&sA[buf][swz(ld_row + 32 * i, ld_chunk)] = ra[i];
    if (BSRC == BSRC_BF16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) *(u32x4_t*)&sB[buf][swz(ld_row + 32 * i, ld_chunk)] = rb[i];
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        *(u32x4_t*)&sB[buf][swz(tid, c)] = dq8(rc[c >> 2][c & 3], ramax, lut);
      }
    }
  };

  auto compute = [&](int buf, int nsub) {
    for (int ks = 0; ks < nsub; ++ks) {
      bf16x8_t a[4], b[4];
      const int ch = 2 * ks + (lane >> 5);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        a[mt] = *(const bf16x8_t*)&sA[buf][swz(wm * 128 + mt * 32 + (lane & 31), ch)];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        b[nt] = *(const bf16x8_t*)&sB[buf][swz(wn * 128 + nt * 32 + (lane & 31), ch)];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
    }
  };

  if (BSRC != BSRC_BF16) __syncthreads();  // lut visible

  // ---- main K loop: two LDS stages, next step's global loads in flight ----
  load_main(0);
  store_main(0);
  __syncthreads();
  for (int kt = 0; kt < nk_main; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk_main;
    if (more) load_main(kt + 1);
    compute(cur, 4);
    if (more) store_main(cur ^ 1);
    __syncthreads();
  }

  // ---- K-extension (LoRA up-projection), bf16 both sides ----
  for (int e = 0; e < nk_ext; ++e) {
    const int c0 = e * BK;
    const int cols = min(BK, p.KE - c0);
    const int nch = cols >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int ga = min(m0 + ld_row + 32 * i, p.M - 1);
      int gb = min(n0 + ld_row + 32 * i, p.N - 1);
      u32x4_t za = {0u, 0u, 0u, 0u}, zb = {0u, 0u, 0u, 0u};
      if (ld_chunk < nch) {
        za = *(const u32x4_t*)(p.Ae + (int64_t)ga * p.ldae + c0 + ld_chunk * 8);
        zb = *(const u32x4_t*)(p.Be + (int64_t)gb * p.ldbe + c0 + ld_chunk * 8);
      }
      *(u32x4_t*)&sA[0][swz(ld_row + 32 * i, ld_chunk)] = za;
      *(u32x4_t*)&sB[0][swz(ld_row + 32 * i, ld_chunk)] = zb;
    }
    __syncthreads();
    compute(0, (cols + 15) >> 4);
    __syncthreads();
  }

  // ---- epilogue ----
  // acc[mt][nt][v] holds C[row][col] with
  //   row = wm*128 + mt*32 + 8*(v/4) + 4*(lane/32) + v%4,  col = wn*128 + nt*32 + lane%32.
  // Each 32-row slab (one mt) of a wave's 128 x 128 tile goes through LDS
  // (fp32, padded pitch) so that the global side moves 16 contiguous bytes
  // per lane; register indices stay compile-time constants.
  constexpr int SP = 136;  // floats per staged row: 4*SP = 32 mod 64 banks
  float* stage = reinterpret_cast<float*>(smem) + wave * (32 * SP);
  const int row0 = m0 + wm * 128;
  const int col0 = n0 + wn * 128;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        stage[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * SP + nt * 32 + (lane & 31)] = acc[mt][nt][v];
    __syncthreads();
    if (EPI == EPI_STORE) {
      // lane: 8 consecutive columns of one row per step, 4 rows per step
      const int cc = (lane & 15) * 8;
      for (int q = 0; q < 8; ++q) {
        const int rr = q * 4 + (lane >> 4);
        const int row = row0 + mt * 32 + rr;
        const int col = col0 + cc;
        const f32x4_t x0 = *(const f32x4_t*)&stage[rr * SP + cc];
        const f32x4_t x1 = *(const f32x4_t*)&stage[rr * SP + cc + 4];
        if (row < p.M && col < p.N) {
          u32x4_t o;
          o[0] = pack_bf16x2(x0[0], x0[1]);
          o[1] = pack_bf16x2(x0[2], x0[3]);
          o[2] = pack_bf16x2(x1[0], x1[1]);
          o[3] = pack_bf16x2(x1[2], x1[3]);
          *(u32x4_t*)(p.C + (int64_t)row * p.ldc + col) = o;
        }
      }
    } else if (EPI == EPI_GATEUP) {
      // staged columns: [gate j0..j0+31 | up j0.. | gate j0+32.. | up j0+32..]
      const int jj = (lane & 7) * 8;
      const int blk = jj >> 5, w = jj & 31;
      const int64_t j = (int64_t)(col0 >> 1) + jj;
      for (int q = 0; q < 4; ++q) {
        const int rr = q * 8 + (lane >> 3);
        const int row = row0 + mt * 32 + rr;
        const float* gs = &stage[rr * SP + blk * 64 + w];
        const float* us = gs + 32;
        if (row < p.M && col0 < p.N) {
          u32x4_t og, ou, oh;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float hv[2];
            uint32_t gb[2], ub[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              gb[t] = f32_to_bf16(gs[2 * e + t]);
              ub[t] = f32_to_bf16(us[2 * e + t]);
              hv[t] = act_fwd(p.act, bf16_to_f32(gb[t])) * bf16_to_f32(ub[t]);
            }
            og[e] = gb[0] | (gb[1] << 16);
            ou[e] = ub[0] | (ub[1] << 16);
            oh[e] = pack_bf16x2(hv[0], hv[1]);
          }
          const int64_t o = (int64_t)row * p.hdim + j;
          *(u32x4_t*)(p.g_out + o) = og;
          *(u32x4_t*)(p.u_out + o) = ou;
          *(u32x4_t*)(p.h_out + o) = oh;
        }
      }
    } else {  // EPI_ACT_BWD: staged values are dH
      const int cc = (lane & 15) * 8;
      for (int q = 0; q < 8; ++q) {
        const int rr = q * 4 + (lane >> 4);
        const int row = row0 + mt * 32 + rr;
        const int col = col0 + cc;
        if (row < p.M && col < p.N) {
          const int64_t o = (int64_t)row * p.hdim + col;
          const u32x4_t gw = *(const u32x4_t*)(p.g_in + o);
          const u32x4_t uw = *(const u32x4_t*)(p.u_in + o);
          const float* dh = &stage[rr * SP + cc];
          u32x4_t odg, odu;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float dg[2], du[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const float g = bf16_to_f32(t ? (gw[e] >> 16) : (gw[e] & 0xFFFFu));
              const float u = bf16_to_f32(t ? (uw[e] >> 16) : (uw[e] & 0xFFFFu));
              float a, da;
              act_fwd_bwd(p.act, g, &a, &da);
              const float d = dh[2 * e + t];
              dg[t] = d * u * da;
              du[t] = d * a;
            }
            odg[e] = pack_bf16x2(dg[0], dg[1]);
            odu[e] = pack_bf16x2(du[0], du[1]);
          }
          const int64_t od = (int64_t)row * (2 * p.hdim) + col;
          *(u32x4_t*)(p.dgu + od) = odg;
          *(u32x4_t*)(p.dgu + od + p.hdim) = odu;
        }
      }
    }
    __syncthreads();
  }
}

template <int BSRC, int EPI>
static hipError_t launch_t(const GemmArgs& a, hipStream_t stream) {
  const int ntm = (a.M + BM - 1) / BM, ntn = (a.N + BN - 1) / BN;
  gemm_nt_kernel<BSRC, EPI><<<dim3(ntm * ntn), dim3(NTHR), 0, stream>>>(a);
  return hipGetLastError();
}

template <int BSRC>
static hipError_t launch_b(const GemmArgs& a, hipStream_t stream) {
  switch (a.epi) {
    case EPI_STORE: return launch_t<BSRC, EPI_STORE>(a, stream);
    case EPI_GATEUP: return launch_t<BSRC, EPI_GATEUP>(a, stream);
    case EPI_ACT_BWD: return launch_t<BSRC, EPI_ACT_BWD>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  switch (a.bsrc) {
    case BSRC_BF16: return launch_b<BSRC_BF16>(a, stream);
    case BSRC_NF4: return launch_b<BSRC_NF4>(a, stream);
    case BSRC_NF4_PAIR: return launch_b<BSRC_NF4_PAIR>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qlora
