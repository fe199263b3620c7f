// The layer around the GDN core: the Gemma-form RMSNorm of the layer input
// and the three linear projections (in_proj_qkvz, in_proj_ba, out_proj).
//
// LightLLM #1097 "[model] Support Qwen3next" lists a Gemma RMSNorm kernel next
// to the GDN kernels ("Specialized Triton Kernels"); the projections are the
// layer's in_proj_qkvz / in_proj_ba and out_proj.  The Gemma form multiplies
// by (1 + w):  out = x / sqrt(mean(x^2) + eps) * (1 + w)  per row.
//
// Projections.  Y[m, n] = sum_k X[m, k] W[n, k] with bf16 operands, fp32
// accumulation and one RNE rounding of the result: a dense contraction, so it
// runs on MFMA (v_mfma_f32_16x16x32_bf16).  Both operands are read along k
// (X rows, weight rows in [out_features, in_features] layout), 64 k per stage
// through LDS.  The MFMA's first operand is the weight tile, so each lane's
// four accumulator values are four consecutive output columns of one row
// (one 8-byte store).  A workgroup owns a BM x BN output tile; each of its
// waves a (BM/WGM) x (BN/WGN) sub-tile held as 16x16 accumulators.  Two
// kernels: one stages each 64-deep step through registers (the next step's
// global loads are issued before the current step's MFMAs, so HBM latency
// hides behind the contraction; two workgroups per CU), the other moves the
// steps straight from HBM into LDS.
//
// LDS rows are 64 bf16 = 128 bytes = 8 chunks of 16 bytes, stored swizzled
// (chunk c of row r at a position that depends on r) so that the rows one
// fragment read touches at one logical chunk spread over the banks.
//
// Workgroup b runs on XCD b % 8; tiles are numbered so that each XCD takes a
// contiguous range, and within that range GM m-tiles share each weight tile
// while it is hot in that XCD's L2.
//
// Output columns may be split over up to four destinations (in_proj writes the
// packed conv input, z, b and a to separate arrays); out_proj may add a
// residual.
#include <hip/hip_runtime.h>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

// ----------------------------------------------------------- Gemma RMSNorm
// One wave per row; two passes over the row (the second hits cache).
template <typename T>
__global__ __launch_bounds__(256) void gemma_norm_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                          float eps, T* __restrict__ out, int64_t rows,
                                                          int hidden) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const T* xr = x + row * hidden;
  T* orow = out + row * hidden;
  const int nch = hidden >> 3;
  float ss = 0.0f;
  for (int c = lane; c < nch; c += 64) {
    float v[8];
    load8(xr + c * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)hidden + eps);
  for (int c = lane; c < nch; c += 64) {
    float v[8], g[8];
    load8(xr + c * 8, v);
    load8(w + c * 8, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * r * (1.0f + g[e]);
    store8(orow + c * 8, v);
  }
}

// ------------------------------------------------------------- projections
constexpr int kBK = 64;  // k per LDS stage (one 128-byte row per tile row)

struct ProjDev {
  const bf16* x;
  int64_t ldx, m;
  const bf16* w0;  // weight rows [0, n_w0)
  const bf16* w1;  // weight rows [n_w0, n)
  int n_w0, n, k;
  int nseg;
  int64_t seg_begin[4];
  bf16* seg_ptr[4];
  int64_t seg_ld[4];
  const bf16* res;
  int64_t ld_res;
  int n_begin;  // first output column of this launch (its tiles cover [n_begin, n))
  int tiles_m, tiles_n, per_xcd, group_m;
};

// One 16-byte global -> LDS transfer per lane (global_load_lds_dwordx4): lane l
// writes bytes [16 l, 16 l + 16) after the wave-uniform LDS address.  Kept out
// of the kernel templates: a target builtin in a template body leaves the
// host-side launch stub of its instantiations undefined.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// Four 16-byte fragments from LDS, waited for inside the asm block, so their
// registers hold the data when it ends.  Written in asm for the direct-to-LDS
// kernel: the compiler cannot tell an LDS read of the current stage from the
// destinations of the next stage's direct-to-LDS loads, and before such a
// read it waits for every load in flight (vmcnt 0), which leaves the next
// stage's loads no MFMA work to overlap.  Stage order is kept by the kernel's
// own wait and barrier at the top of each stage.
__device__ __forceinline__ uint32_t lds_addr(const bf16* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) bf16*)p;
}
__device__ __forceinline__ void lds_read4(const bf16* p0, const bf16* p1, const bf16* p2, const bf16* p3,
                                          bf16x8& o0, bf16x8& o1, bf16x8& o2, bf16x8& o3) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3)
      : "v"(lds_addr(p0)), "v"(lds_addr(p1)), "v"(lds_addr(p2)), "v"(lds_addr(p3))
      : "memory");
}

// Register-staged kernel: chunk c of row r at c ^ (r % 8).
__device__ __forceinline__ int swz(int row, int c) { return row * kBK + ((c ^ (row & 7)) << 3); }

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ int seg_of(const ProjDev& p, int64_t n) {
  int s = 0;
#pragma unroll
  for (int q = 1; q < 4; ++q)
    if (q < p.nseg && n >= p.seg_begin[q]) s = q;
  return s;
}

// Writes a wave's accumulators: lane (rl, g) of 16x16 tile (j, i) holds output
// columns n .. n+3 (n = nb + 16 j + 4 g) of row m = mb + 16 i + rl.  VEC: every
// segment starts at a multiple of 4 columns with a row stride that is one too,
// and n is one: four columns always share a segment (one 8-byte store).
// Otherwise one column at a time.
template <bool VEC, bool RES, int FN, int FM>
__device__ __forceinline__ void store_tile(const ProjDev& p, int64_t mb, int nb, int rl, int g,
                                           const f32x4 (&acc)[FN][FM]) {
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = nb + j * 16 + 4 * g;
    if (n >= p.n) continue;
    if constexpr (VEC) {
      const int s = seg_of(p, n);
      bf16* base = p.seg_ptr[s] + (n - p.seg_begin[s]);
      const int64_t ld = p.seg_ld[s];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t m = mb + i * 16 + rl;
        if (m >= p.m) continue;
        float o0 = acc[j][i][0], o1 = acc[j][i][1], o2 = acc[j][i][2], o3 = acc[j][i][3];
        if constexpr (RES) {
          const uint2 r = *reinterpret_cast<const uint2*>(p.res + m * p.ld_res + n);
          o0 += bf_lo(r.x);
          o1 += bf_hi(r.x);
          o2 += bf_lo(r.y);
          o3 += bf_hi(r.y);
        }
        const bf16x4 b = {(bf16)o0, (bf16)o1, (bf16)o2, (bf16)o3};
        *reinterpret_cast<bf16x4*>(base + m * ld) = b;
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t m = mb + i * 16 + rl;
        if (m >= p.m) continue;
        for (int e = 0; e < 4; ++e) {
          const int ne = n + e;
          if (ne >= p.n) break;
          const int se = seg_of(p, ne);
          float o = acc[j][i][e];
          if constexpr (RES) o += (float)p.res[m * p.ld_res + ne];
          p.seg_ptr[se][m * p.seg_ld[se] + (ne - p.seg_begin[se])] = (bf16)o;
        }
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int OCC, bool VEC, bool RES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void proj_kernel(ProjDev p) {
  static_assert(WGM * WGN == 4, "four waves");
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 16, FN = WN / 16;
  constexpr int LX = BM / 32, LW = BN / 32;  // 16-byte chunks per thread per stage
  static_assert(WM % 16 == 0 && WN % 16 == 0 && BM % 32 == 0 && BN % 32 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) bf16 sx[BM * kBK];
  __shared__ __attribute__((aligned(16))) bf16 sw[BN * kBK];

  // tile order: XCD-contiguous ranges, then groups of group_m m-tiles per n-tile
  const int b = blockIdx.x;
  const int64_t lt = (int64_t)(b & 7) * p.per_xcd + (b >> 3);
  if (lt >= (int64_t)p.tiles_m * p.tiles_n) return;
  const int64_t span = (int64_t)p.group_m * p.tiles_n;
  const int grp = (int)(lt / span);
  const int gm = min(p.group_m, p.tiles_m - grp * p.group_m);
  const int within = (int)(lt - grp * span);
  const int mt = grp * p.group_m + within % gm;
  const int nt = within / gm;
  const int64_t m0 = (int64_t)mt * BM;
  const int n0 = p.n_begin + nt * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ch = tid & 7, r0 = tid >> 3;
  const bf16* xs[LX];
  const bf16* ws[LW];
#pragma unroll
  for (int i = 0; i < LX; ++i) {
    const int64_t row = m0 + r0 + 32 * i;
    xs[i] = row < p.m ? p.x + row * p.ldx + ch * 8 : nullptr;
  }
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const int n = n0 + r0 + 32 * i;
    ws[i] = n < p.n_w0 ? p.w0 + (int64_t)n * p.k + ch * 8
                       : (n < p.n ? p.w1 + (int64_t)(n - p.n_w0) * p.k + ch * 8 : nullptr);
  }
  uint4 rx[LX], rw[LW];
  auto gload = [&](int k0) {
    const bool kin = k0 + ch * 8 < p.k;
#pragma unroll
    for (int i = 0; i < LX; ++i)
      rx[i] = (xs[i] && kin) ? *reinterpret_cast<const uint4*>(xs[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < LW; ++i)
      rw[i] = (ws[i] && kin) ? *reinterpret_cast<const uint4*>(ws[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < LX; ++i) *reinterpret_cast<uint4*>(&sx[swz(r0 + 32 * i, ch)]) = rx[i];
#pragma unroll
    for (int i = 0; i < LW; ++i) *reinterpret_cast<uint4*>(&sw[swz(r0 + 32 * i, ch)]) = rw[i];
  };

  const int wm = wave % WGM, wn = wave / WGM;
  const int rl = lane & 15, g = lane >> 4;
  f32x4 acc[FN][FM];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[j][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int kt_n = (p.k + kBK - 1) / kBK;
  gload(0);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < kt_n; ++kt) {
    if (kt + 1 < kt_n) gload((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + g;
      bf16x8 fw[FN], fx[FM];
#pragma unroll
      for (int j = 0; j < FN; ++j) fw[j] = *reinterpret_cast<const bf16x8*>(&sw[swz(wn * WN + j * 16 + rl, c)]);
#pragma unroll
      for (int i = 0; i < FM; ++i) fx[i] = *reinterpret_cast<const bf16x8*>(&sx[swz(wm * WM + i * 16 + rl, c)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[j], fx[i], acc[j][i], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < kt_n) {
      sstore();
      __syncthreads();
    }
  }

  store_tile<VEC, RES, FN, FM>(p, m0 + wm * WM, n0 + wn * WN, rl, g, acc);
}

// The same contraction for k a multiple of 64, with the stages moved from HBM
// straight into LDS (global_load_lds_dwordx4: no staging registers, no LDS
// store instructions), 4 or 8 waves (one or two per SIMD) and two LDS
// buffers, so the next stage streams in while
// the MFMAs consume the current one; one barrier per stage.  A wave's load
// instruction fills one contiguous kilobyte of LDS (lane l: bytes 16 l), i.e.
// 8 tile rows: lane l writes physical chunk l % 8 of row l / 8 and so fetches
// the logical chunk that the swizzle puts there.  Rows past m or n read the
// last valid row instead (in bounds; their outputs are never stored).  Weight
// rows from n_w0 on come from the second weight matrix, as in the kernel above.
//
// The swizzle here is chunk c of row r at c ^ ((r / 2) % 8): the 16 rows a
// quarter-wave reads at one logical chunk then cover all 64 banks once.
__device__ __forceinline__ int swz2(int row, int c) { return row * kBK + ((c ^ ((row >> 1) & 7)) << 3); }

template <int BM, int BN, int WGM, int WGN, bool RES, int NBUF = 2>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(WGM * WGN / 4, WGM * WGN / 4)))
void proj_lds_kernel(ProjDev p) {
  constexpr int NW = WGM * WGN;  // waves: 4 (one per SIMD) or 8 (two per SIMD)
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 16, FN = WN / 16;
  static_assert(FM * 16 == WM && FN * 16 == WN, "wave tile");
  static_assert(FM % 4 == 0 && FN % 4 == 0, "fragments read four at a time");
  constexpr int IX = BM / (8 * NW), IW = BN / (8 * NW);  // load instructions per wave per stage
  static_assert(IX * 8 * NW == BM && IW * 8 * NW == BN, "whole load instructions");
  // NBUF LDS buffers: NBUF - 1 stages in flight while one is consumed; a
  // wave's loads of stage kt have landed once at most the later stages' loads
  // are outstanding (loads retire in issue order; no other memory operation
  // is issued in the k loop)
  static_assert(NBUF >= 2 && (NBUF - 2) * (IX + IW) < 64, "stages in flight");
  constexpr int VM_LATER = (NBUF - 2) * (IX + IW);
  constexpr int WAIT_KT = 0x0F70 | (VM_LATER & 15) | ((VM_LATER >> 4) << 14);  // vmcnt(VM_LATER)
  __shared__ __attribute__((aligned(16))) bf16 sx[NBUF][BM * kBK];
  __shared__ __attribute__((aligned(16))) bf16 sw[NBUF][BN * kBK];

  const int b = blockIdx.x;
  const int64_t lt = (int64_t)(b & 7) * p.per_xcd + (b >> 3);
  if (lt >= (int64_t)p.tiles_m * p.tiles_n) return;
  const int64_t span = (int64_t)p.group_m * p.tiles_n;
  const int grp = (int)(lt / span);
  const int gm = min(p.group_m, p.tiles_m - grp * p.group_m);
  const int within = (int)(lt - grp * span);
  const int mt = grp * p.group_m + within % gm;
  const int nt = within / gm;
  const int64_t m0 = (int64_t)mt * BM;
  const int n0 = p.n_begin + nt * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane >> 3;
  // each lane's row addresses, fixed for the whole k loop (computed once from
  // scalar copies of the pointers: a per-lane choice between two pointers of
  // the argument block would otherwise become a per-lane load of the pointer)
  const bf16* const xbase = p.x;
  const bf16* const w0 = p.w0;
  const bf16* const w1 = p.w1;
  const bf16* xrow[IX];
  const bf16* wrow[IW];
  auto lchunk = [&](int blk) { return (lane & 7) ^ (((blk * 8 + lrow) >> 1) & 7); };
#pragma unroll
  for (int i = 0; i < IX; ++i) {
    const int blk = i * NW + wave;
    const int64_t row = min(m0 + blk * 8 + lrow, p.m - 1);
    xrow[i] = xbase + row * p.ldx + lchunk(blk) * 8;
  }
#pragma unroll
  for (int i = 0; i < IW; ++i) {
    const int blk = i * NW + wave;
    const int n = min(n0 + blk * 8 + lrow, p.n - 1);
    const int64_t off = n < p.n_w0 ? (int64_t)n * p.k : (int64_t)(n - p.n_w0) * p.k;
    wrow[i] = (n < p.n_w0 ? w0 : w1) + off + lchunk(blk) * 8;
  }
  auto issue = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < IX; ++i) lds_dma16(xrow[i] + k0, &sx[buf][(i * NW + wave) * 8 * kBK]);
#pragma unroll
    for (int i = 0; i < IW; ++i) lds_dma16(wrow[i] + k0, &sw[buf][(i * NW + wave) * 8 * kBK]);
  };

  const int wm = wave % WGM, wn = wave / WGM;
  f32x4 acc[FN][FM];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[j][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // fragments: lane l reads row l % 16 at chunk 4 kk + l / 16 (two 32-deep
  // steps per stage)
  const int rl = lane & 15, g = lane >> 4;
  const int kt_n = p.k / kBK;
  // stages 0 .. NBUF-2 up front; no load is ever issued past the end of k,
  // so none is in flight when the workgroup ends
#pragma unroll
  for (int q = 0; q < NBUF - 1; ++q)
    if (q < kt_n) issue(q * kBK, q);
  for (int kt = 0; kt < kt_n; ++kt) {
    const int buf = kt % NBUF;
    // this wave's loads of stage kt have landed: with all NBUF - 2 later
    // stages issued, at most their loads are outstanding; near the end, none
    if (kt + NBUF - 2 < kt_n) __builtin_amdgcn_s_waitcnt(WAIT_KT);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    // ... everyone's, and everyone is done reading stage kt - 1 (the asm reads
    // retire before their block ends).  A bare barrier: __syncthreads' fence
    // would also wait for the later stages' loads (it counts direct-to-LDS
    // loads as pending LDS writes) and drain the pipeline
    asm volatile("s_barrier" ::: "memory");
    if (kt + NBUF - 1 < kt_n) issue((kt + NBUF - 1) * kBK, (kt + NBUF - 1) % NBUF);
    const bf16* cx = sx[buf];
    const bf16* cw = sw[buf];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + g;
      bf16x8 fx[FM], fw[FN];
      auto xp = [&](int i) { return &cx[swz2(wm * WM + i * 16 + rl, c)]; };
      auto wp = [&](int j) { return &cw[swz2(wn * WN + j * 16 + rl, c)]; };
#pragma unroll
      for (int i = 0; i < FM; i += 4) lds_read4(xp(i), xp(i + 1), xp(i + 2), xp(i + 3), fx[i], fx[i + 1], fx[i + 2], fx[i + 3]);
#pragma unroll
      for (int j = 0; j < FN; j += 4) lds_read4(wp(j), wp(j + 1), wp(j + 2), wp(j + 3), fw[j], fw[j + 1], fw[j + 2], fw[j + 3]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[j], fx[i], acc[j][i], 0, 0, 0);
    }
  }

  store_tile<true, RES, FN, FM>(p, m0 + wm * WM, n0 + wn * WN, rl, g, acc);
}

// Few rows (decode): the contraction of a BM x BN tile is split over k
// between the four waves (wave w takes the w-th quarter of k), so each wave's
// serial loop is a quarter as long; every wave holds the whole tile's
// accumulators and reads its MFMA fragments straight from global memory into
// registers, PD 64-deep stages in flight, with no LDS staging and no barrier
// in the loop.  The four partial tiles are then summed through LDS in wave
// order and stored as the other kernels store theirs.  k is a multiple of 256.
template <int BM, int BN, int PD, bool RES>
__global__ __launch_bounds__(256) void proj_splitk_kernel(ProjDev p) {
  constexpr int FM = BM / 16, FN = BN / 16, T = FM * FN;
  static_assert(PD >= 2, "stages");
  __shared__ __attribute__((aligned(16))) f32x4 red[4][T][64];

  const int b = blockIdx.x;
  const int64_t lt = (int64_t)(b & 7) * p.per_xcd + (b >> 3);
  if (lt >= (int64_t)p.tiles_m * p.tiles_n) return;
  const int64_t span = (int64_t)p.group_m * p.tiles_n;
  const int grp = (int)(lt / span);
  const int gm = min(p.group_m, p.tiles_m - grp * p.group_m);
  const int within = (int)(lt - grp * span);
  const int mt = grp * p.group_m + within % gm;
  const int nt = within / gm;
  const int64_t m0 = (int64_t)mt * BM;
  const int n0 = p.n_begin + nt * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = lane & 15, g = lane >> 4;
  // this lane's rows (clamped to the last valid one: in bounds, never stored)
  const bf16* const xbase = p.x;
  const bf16* const w0 = p.w0;
  const bf16* const w1 = p.w1;
  const int kq = p.k / 4;                            // this wave's k range [wave kq, wave kq + kq)
  const bf16* xr[FM];
  const bf16* wr[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = min(m0 + 16 * i + rl, p.m - 1);
    xr[i] = xbase + row * p.ldx + wave * kq + 8 * g;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = min(n0 + 16 * j + rl, p.n - 1);
    wr[j] = (n < p.n_w0 ? w0 + (int64_t)n * p.k : w1 + (int64_t)(n - p.n_w0) * p.k) + wave * kq + 8 * g;
  }
  // stage st, half kk: logical chunk kk * 4 + g of the 64-deep step, as in the
  // LDS-staged kernels
  bf16x8 fx[PD][2][FM], fw[PD][2][FN];
  auto load = [&](int s, int st) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int k = st * kBK + kk * 32;
#pragma unroll
      for (int i = 0; i < FM; ++i) fx[s][kk][i] = *reinterpret_cast<const bf16x8*>(xr[i] + k);
#pragma unroll
      for (int j = 0; j < FN; ++j) fw[s][kk][j] = *reinterpret_cast<const bf16x8*>(wr[j] + k);
    }
  };
  f32x4 acc[FN][FM];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[j][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int ns = kq / kBK;
#pragma unroll
  for (int s = 0; s < PD - 1; ++s)
    if (s < ns) load(s, s);
  for (int st0 = 0; st0 < ns; st0 += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int st = st0 + s;
      if (st < ns) {  // (uniform)
        if (st + PD - 1 < ns) load((s + PD - 1) % PD, st + PD - 1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i)
              acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[s][kk][j], fx[s][kk][i], acc[j][i], 0, 0, 0);
      }
    }
  }
  // partial tiles -> LDS; wave w sums tiles w, w + 4, ... over the waves in order
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int i = 0; i < FM; ++i) red[wave][j * FM + i][lane] = acc[j][i];
  __syncthreads();
  for (int t = wave; t < T; t += 4) {
    f32x4 v = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 q = red[w][t][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += q[e];
    }
    const int j = t / FM, i = t % FM;
    const int n = n0 + 16 * j + 4 * g;
    const int64_t m = m0 + 16 * i + rl;
    if (n >= p.n || m >= p.m) continue;
    const int sg = seg_of(p, n);
    float o0 = v[0], o1 = v[1], o2 = v[2], o3 = v[3];
    if constexpr (RES) {
      const uint2 r = *reinterpret_cast<const uint2*>(p.res + m * p.ld_res + n);
      o0 += bf_lo(r.x);
      o1 += bf_hi(r.x);
      o2 += bf_lo(r.y);
      o3 += bf_hi(r.y);
    }
    const bf16x4 o = {(bf16)o0, (bf16)o1, (bf16)o2, (bf16)o3};
    *reinterpret_cast<bf16x4*>(p.seg_ptr[sg] + (n - p.seg_begin[sg]) + m * p.seg_ld[sg]) = o;
  }
}

template <int BM, int BN, int PD, bool RES>
hipError_t run_proj_splitk(ProjDev p, hipStream_t st) {
  p.tiles_m = (int)((p.m + BM - 1) / BM);
  p.tiles_n = (p.n - p.n_begin + BN - 1) / BN;
  p.group_m = 4;
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  p.per_xcd = (int)((tiles + 7) / 8);
  hipLaunchKernelGGL((proj_splitk_kernel<BM, BN, PD, RES>), dim3((unsigned)(8 * (int64_t)p.per_xcd)), dim3(256), 0,
                     st, p);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, bool RES, int NBUF = 2>
hipError_t run_proj_lds(ProjDev p, hipStream_t st) {
  p.tiles_m = (int)((p.m + BM - 1) / BM);
  p.tiles_n = (p.n - p.n_begin + BN - 1) / BN;
  p.group_m = 4;
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  p.per_xcd = (int)((tiles + 7) / 8);
  hipLaunchKernelGGL((proj_lds_kernel<BM, BN, WGM, WGN, RES, NBUF>), dim3((unsigned)(8 * (int64_t)p.per_xcd)),
                     dim3(64 * WGM * WGN), 0, st, p);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int OCC, bool VEC, bool RES>
hipError_t run_proj(ProjDev p, hipStream_t st) {
  p.tiles_m = (int)((p.m + BM - 1) / BM);
  p.tiles_n = (p.n - p.n_begin + BN - 1) / BN;
  p.group_m = 4;
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  p.per_xcd = (int)((tiles + 7) / 8);
  hipLaunchKernelGGL((proj_kernel<BM, BN, WGM, WGN, OCC, VEC, RES>), dim3((unsigned)(8 * (int64_t)p.per_xcd)),
                     dim3(256), 0, st, p);
  return hipGetLastError();
}

int64_t tile_count(int64_t m, int n, int bm, int bn) { return ((m + bm - 1) / bm) * ((n + bn - 1) / bn); }

}  // namespace

hipError_t launch_gemma_norm(const GemmaNormArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
  if (a.bf16)
    hipLaunchKernelGGL(gemma_norm_kernel<bf16>, grid, block, 0, st, (const bf16*)a.x, (const bf16*)a.w, a.eps,
                       (bf16*)a.out, a.rows, a.hidden);
  else
    hipLaunchKernelGGL(gemma_norm_kernel<float>, grid, block, 0, st, (const float*)a.x, (const float*)a.w, a.eps,
                       (float*)a.out, a.rows, a.hidden);
  return hipGetLastError();
}

hipError_t launch_proj(const ProjArgs& a, hipStream_t st) {
  ProjDev p{};
  p.x = (const bf16*)a.x;
  p.ldx = a.ldx;
  p.m = a.m;
  p.w0 = (const bf16*)a.w0;
  p.w1 = (const bf16*)a.w1;
  p.n_w0 = a.n_w0;
  p.n = a.n;
  p.k = a.k;
  p.nseg = a.nseg;
  for (int s = 0; s < 4; ++s) {
    p.seg_begin[s] = s < a.nseg ? a.seg[s].begin : a.n;
    p.seg_ptr[s] = s < a.nseg ? (bf16*)a.seg[s].ptr : nullptr;
    p.seg_ld[s] = s < a.nseg ? a.seg[s].ld : 0;
  }
  p.res = (const bf16*)a.residual;
  p.ld_res = a.ld_res;
  // four output columns per lane store at once when every segment allows it
  bool vec = a.n % 4 == 0 && (a.residual == nullptr || (a.ld_res % 4 == 0 && ((uintptr_t)a.residual & 7) == 0));
  for (int s = 0; s < a.nseg; ++s)
    vec = vec && a.seg[s].begin % 4 == 0 && a.seg[s].ld % 4 == 0 && ((uintptr_t)a.seg[s].ptr & 7) == 0;
  // Measured on the layer's shapes (hidden 2048): at 4096 tokens
  // in_proj_qkvz/ba runs best as 256 x 256 tiles streamed straight into LDS
  // (8 waves, two per SIMD, two LDS buffers) and out_proj (k = 4096: 64
  // stages) as 128 x 256 tiles streamed into three LDS buffers, two stages in
  // flight; at 256 decode rows in_proj takes 64 x 128 tiles and out_proj
  // 64 x 32.
  const bool lds = vec && a.k % kBK == 0;
  const bool res = a.residual != nullptr;
  if (lds && !res && a.m >= 1024 && tile_count(a.m, a.n, 256, 256) >= 512) {
    // A narrow last column tile (in_proj's 2 h_v columns of b and a past
    // 48 tiles of 256) would cost a whole round of 256 x 256 tiles on its
    // own: those columns go to a second launch of small register-staged tiles.
    const int n_full = a.n / 256 * 256;
    if (n_full == a.n || a.n - n_full > 128) return run_proj_lds<256, 256, 2, 4, false>(p, st);
    ProjDev rest = p;
    p.n = n_full;
    if (hipError_t e = run_proj_lds<256, 256, 2, 4, false>(p, st); e != hipSuccess) return e;
    rest.n_begin = n_full;
    return run_proj<64, 32, 2, 2, 2, true, false>(rest, st);
  }
  if (lds && res && a.m >= 1024 && tile_count(a.m, a.n, 128, 256) >= 256)
    return run_proj_lds<128, 256, 2, 4, true, 3>(p, st);
  // few rows and few columns (a decode step's out_proj): k split over the
  // waves; with many columns (in_proj) the LDS-staged tiles below share each
  // weight stage between the waves and run faster
  if (vec && a.k % 256 == 0 && a.m <= 512 && tile_count(a.m, a.n, 64, 128) < 256)
    return res ? run_proj_splitk<64, 32, 3, true>(p, st) : run_proj_splitk<64, 32, 3, false>(p, st);
#define GDN_PROJ(BM_, BN_, WGM_, WGN_)                                                              \
  do {                                                                                               \
    if (vec)                                                                                         \
      return res ? run_proj<BM_, BN_, WGM_, WGN_, 2, true, true>(p, st)                               \
                 : run_proj<BM_, BN_, WGM_, WGN_, 2, true, false>(p, st);                             \
    return res ? run_proj<BM_, BN_, WGM_, WGN_, 2, false, true>(p, st)                                \
               : run_proj<BM_, BN_, WGM_, WGN_, 2, false, false>(p, st);                              \
  } while (0)
  // otherwise the largest register-staged tile that still gives 256
  // workgroups: a small m (decode) is bound by per-step overheads of each
  // workgroup's k loop, so more, smaller tiles run faster there
  if (tile_count(a.m, a.n, 128, 128) >= 256) GDN_PROJ(128, 128, 2, 2);
  if (tile_count(a.m, a.n, 64, 128) >= 256) GDN_PROJ(64, 128, 1, 4);
  if (tile_count(a.m, a.n, 64, 64) >= 256) GDN_PROJ(64, 64, 2, 2);
  GDN_PROJ(64, 32, 2, 2);
#undef GDN_PROJ
}

}  // namespace gdn
