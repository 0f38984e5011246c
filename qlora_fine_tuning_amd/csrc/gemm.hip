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
// Tiling: 256 x 256 output tile per workgroup of 8 waves (2 per SIMD) laid
// out 2 x 4, each wave 128 x 64 = 4 x 2 MFMA 32x32x16 tiles (128 fp32
// accumulators per lane). Two waves per SIMD let one wave's LDS or barrier
// wait be covered by the other's matrix work. K is walked in 32-wide steps
// through a 4-deep LDS ring (4 x 32 KB of the 160 KB per CU) filled by
// direct-to-LDS loads (global_load_lds_dwordx4) issued three steps ahead, so
// operands never pass through VGPRs. LDS rows are 64 B; the 16-byte chunk
// index is XOR-swizzled with ((row >> 1) ^ (row >> 3)) & 3, which keeps
// every 16-lane phase of a ds_read_b128 fragment load (and every 8-lane one)
// on distinct banks.
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

constexpr int BM = 256, BN = 256, BK = 32, NTHR = 512, NWAVE = 8;
constexpr int NSTAGE = 4;          // LDS ring depth
constexpr int PREF = NSTAGE - 1;   // k-tiles in flight ahead of the one computed

// Per-stage LDS layout (bytes): A [256][32] bf16, B [256][32] bf16, then (NF4
// modes) the raw codes [256][16 B] and one fp32 absmax per B row.
constexpr int A_BYTES = BM * BK * 2;
constexpr int B_BYTES = BN * BK * 2;
constexpr int C_BYTES = BN * 16;
constexpr int S_BYTES = BN * 4;
constexpr int STAGE_BF16 = A_BYTES + B_BYTES;
constexpr int STAGE_NF4 = A_BYTES + B_BYTES + C_BYTES + S_BYTES;

// element offset of (row, 16-byte chunk) in a [rows][32] bf16 LDS tile; see
// the swizzle note above.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (((row >> 1) ^ (row >> 3)) & 3)) << 3);
}

__device__ __forceinline__ int xcd_remap(int pid, int n) {
  const int X = 8;
  int q = n / X, rmd = n % X;
  int xcd = pid % X, local = pid / X;
  return (xcd < rmd ? xcd * (q + 1) : rmd * (q + 1) + (xcd - rmd) * q) + local;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS at base + 16*lane.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 16, 0, 0);
}
// 4 bytes per lane into LDS at base + 4*lane.
__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 4, 0, 0);
}

// Wait until at most N vector-memory loads of this wave are outstanding and
// all of its LDS operations are done (expcnt left unconstrained).
// gfx9 encoding: vmcnt[3:0] | vmcnt[5:4] << 14, expcnt[6:4], lgkmcnt[11:8].
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would wait for every DMA in flight (vmcnt(0)) and drain the LDS ring. The
// waves wait for their own DMA stage with wait_vm<> first, so after the
// barrier every wave's data for that stage is in LDS. The empty asm keeps the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int L>
__device__ __forceinline__ void wait_vm_stages(int later) {
  if (later >= 2) wait_vm<2 * L>();
  else if (later == 1) wait_vm<L>();
  else wait_vm<0>();
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
__global__ __launch_bounds__(NTHR)
void gemm_nt_kernel(GemmArgs p) {
  constexpr bool NF4 = BSRC != BSRC_BF16;
  constexpr int STAGE = NF4 ? STAGE_NF4 : STAGE_BF16;
  constexpr int L = NF4 ? 3 : 4;  // DMA instructions per stage per wave
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * STAGE];
  __shared__ float lut[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  if (NF4) {
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
  const int nk = p.K / BK;

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // ---- per-lane DMA sources (row and swizzled chunk fixed; k advances) ----
  // Tile A/B: wave w, instruction j fills LDS slots (w*2 + j)*64 + lane of
  // the [256][4 x 16 B] tile; slot -> (row, physical chunk) -> logical chunk.
  const uint16_t* srcA[2];
  const uint16_t* srcB[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int slot = (wave * 2 + j) * 64 + lane;
    const int row = slot >> 2, phys = slot & 3;
    const int chunk = phys ^ (((row >> 1) ^ (row >> 3)) & 3);
    srcA[j] = p.A + (int64_t)min(m0 + row, p.M - 1) * p.lda + chunk * 8;
    if (!NF4) srcB[j] = p.B + (int64_t)min(n0 + row, p.N - 1) * p.ldb + chunk * 8;
  }
  // NF4: waves 0-3 move the 16 code bytes of B rows w*64 + lane, waves 4-7
  // the absmax of B rows (w-4)*64 + lane, one k-tile per stage.
  const uint8_t* srcC = nullptr;
  const float* srcS = nullptr;
  if (NF4) {
    const int gn = min(n0 + (wave & 3) * 64 + lane, p.N - 1);
    const uint8_t* codes = p.codes0;
    const float* amax = p.absmax0;
    int64_t wrow = gn;
    if (BSRC == BSRC_NF4_PAIR) {
      const int which = (gn >> 5) & 1;
      wrow = (int64_t)((gn >> 6) << 5) + (gn & 31);
      codes = which ? p.codes1 : p.codes0;
      amax = which ? p.absmax1 : p.absmax0;
    }
    srcC = codes + wrow * (int64_t)(p.K >> 1);
    srcS = amax + wrow * (int64_t)(p.K >> 6);
  }

  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % NSTAGE) * STAGE;
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(srcA[j] + k0, st + (wave * 2 + j) * 1024);
    if (!NF4) {
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16(srcB[j] + k0, st + A_BYTES + (wave * 2 + j) * 1024);
    } else if (wave < 4) {
      dma16(srcC + (k0 >> 1), st + A_BYTES + B_BYTES + wave * 1024);
    } else {
      dma4(srcS + (kt >> 1), st + A_BYTES + B_BYTES + C_BYTES + (wave - 4) * 256);
    }
  };

  // NF4: two threads per B row (16 weights each) dequantize a landed stage
  // into its bf16 region.
  auto dequant_stage = [&](int kt) {
    uint8_t* st = smem + (kt % NSTAGE) * STAGE;
    const int row = tid >> 1, half = tid & 1;
    const u32x2_t w = *(const u32x2_t*)(st + A_BYTES + B_BYTES + row * 16 + half * 8);
    const float amax = *(const float*)(st + A_BYTES + B_BYTES + C_BYTES + row * 4);
    uint16_t* sb = (uint16_t*)(st + A_BYTES);
#pragma unroll
    for (int c = 0; c < 2; ++c) *(u32x4_t*)&sb[swz(row, half * 2 + c)] = dq8(w[c], amax, lut);
  };

  auto compute = [&](const uint8_t* st, int nsub) {
    const uint16_t* sa = (const uint16_t*)st;
    const uint16_t* sb = (const uint16_t*)(st + A_BYTES);
    for (int ks = 0; ks < nsub; ++ks) {
      bf16x8_t a[4], b[2];
      const int ch = 2 * ks + (lane >> 5);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        a[mt] = *(const bf16x8_t*)&sa[swz(wm * 128 + mt * 32 + (lane & 31), ch)];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        b[nt] = *(const bf16x8_t*)&sb[swz(wn * 64 + nt * 32 + (lane & 31), ch)];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
    }
  };

  // ---- main K loop ----
  if (!NF4) {
    // bf16 operands: NSTAGE-deep LDS ring, PREF k-tiles of DMA in flight.
    const int npro = min(PREF, nk);
    for (int kt = 0; kt < npro; ++kt) issue(kt);
    for (int kt = 0; kt < nk; ++kt) {
      wait_vm_stages<L>(min(nk - 1 - kt, PREF - 1));  // this wave's stage kt landed
      ring_barrier();                                 // everyone's stage kt landed; kt-1 consumed
      if (kt + PREF < nk) issue(kt + PREF);
      compute(smem + (kt % NSTAGE) * STAGE, BK / 16);
    }
  } else {
    // NF4 weights: raw codes/absmax arrive by DMA one k-tile ahead and are
    // dequantized in LDS by the block. The in-loop LDS stores are ordered
    // after all DMA in flight, so the raw data runs one stage ahead only.
    issue(0);
    if (nk > 1) issue(1);
    wait_vm_stages<L>(nk > 1 ? 1 : 0);
    ring_barrier();  // stage 0 raw data and lut visible
    dequant_stage(0);
    for (int kt = 0; kt < nk; ++kt) {
      wait_vm<0>();   // stage kt+1 raw data landed (and the dequant stores of stage kt done)
      ring_barrier();
      if (kt + 1 < nk) dequant_stage(kt + 1);
      if (kt + 2 < nk) issue(kt + 2);
      compute(smem + (kt % NSTAGE) * STAGE, BK / 16);
    }
  }
  __syncthreads();

  // ---- K-extension (LoRA up-projection), bf16 both sides, via registers ----
  for (int e = 0; e * BK < p.KE; ++e) {
    const int c0 = e * BK;
    const int nch = min(BK, p.KE - c0) >> 3;
    uint16_t* sa = (uint16_t*)smem;
    uint16_t* sb = (uint16_t*)(smem + A_BYTES);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (tid >> 2) + 128 * i, chunk = tid & 3;
      const int ga = min(m0 + row, p.M - 1), gb = min(n0 + row, p.N - 1);
      u32x4_t za = {0u, 0u, 0u, 0u}, zb = {0u, 0u, 0u, 0u};
      if (chunk < nch) {
        za = *(const u32x4_t*)(p.Ae + (int64_t)ga * p.ldae + c0 + chunk * 8);
        zb = *(const u32x4_t*)(p.Be + (int64_t)gb * p.ldbe + c0 + chunk * 8);
      }
      *(u32x4_t*)&sa[swz(row, chunk)] = za;
      *(u32x4_t*)&sb[swz(row, chunk)] = zb;
    }
    __syncthreads();
    compute(smem, (nch * 8 + 15) >> 4);
    __syncthreads();
  }

  // ---- epilogue ----
  // acc[mt][nt][v] holds C[row][col] with
  //   row = wm*128 + mt*32 + 8*(v/4) + 4*(lane/32) + v%4,  col = wn*64 + nt*32 + lane%32.
  // Each 32-row slab (one mt) of a wave's 128 x 64 tile goes through LDS
  // (fp32, padded pitch) so that the global side moves 16 contiguous bytes
  // per lane; register indices stay compile-time constants.
  constexpr int SP = 72;  // floats per staged row: 4*SP = 32 mod 64 banks
  float* stage = reinterpret_cast<float*>(smem) + wave * (32 * SP);  // fits in the ring
  const int row0 = m0 + wm * 128;
  const int col0 = n0 + wn * 64;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        stage[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * SP + nt * 32 + (lane & 31)] = acc[mt][nt][v];
    __syncthreads();
    if (EPI == EPI_STORE) {
      // lane: 8 consecutive columns of one row per step, 8 rows per step
      const int cc = (lane & 7) * 8;
      for (int q = 0; q < 4; ++q) {
        const int rr = q * 8 + (lane >> 3);
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
      // staged columns: [gate j0..j0+31 | up j0..j0+31], j0 = col0 / 2
      const int jj = (lane & 3) * 8;
      const int64_t j = (int64_t)(col0 >> 1) + jj;
      for (int q = 0; q < 2; ++q) {
        const int rr = q * 16 + (lane >> 2);
        const int row = row0 + mt * 32 + rr;
        const float* gs = &stage[rr * SP + jj];
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
      const int cc = (lane & 7) * 8;
      for (int q = 0; q < 4; ++q) {
        const int rr = q * 8 + (lane >> 3);
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
