// Verify-shaped linear layer on gfx950: y = x W^T.
//
// With speculation every linear layer of the target sees M*(1+D) rows in the
// verify pass instead of M, against the same weight ("Co-Designing AI Models
// Using Speculative Decoding for Faster LLM Inference", translated page,
// section "Draft length and performance of linear layers", Figure 3: an
// expert GEMM of N = K = 6144).  With few rows the product is bound by reading
// W (N*K*2 bytes); from about 312 rows on (2.5 PFLOP/s over 8 TB/s) it is
// bound by the bf16 MFMA rate.
//
// A workgroup computes a BM x BN tile of y (BM = 32, 64, 128 or 256 and
// BN = 128 or 256, chosen by M) over a range of K: 4 waves for the 32- and
// 64-row tiles, 8 (two per SIMD, so that one wave's MFMAs run while the other
// waits at the ring) for the 128- and 256-row tiles, which fill the LDS at one
// workgroup per CU.  x and W tiles of 64 k travel global -> LDS with global_load_lds_dwordx4
// into a ring of S stages, and each wave multiplies 32x32 blocks with
// v_mfma_f32_32x32x16_bf16 (A = rows of x, B = rows of W, both read from LDS
// as 16-byte chunks).  When M
// gives too few tiles to fill the GPU, K is split: each split writes an fp32 partial and a second
// kernel adds the partials in split order (the result does not depend on
// timing) and rounds to bf16.

#include "common.h"

namespace sdv {

constexpr int kGemmBK = 64;              // k per ring stage
constexpr int kGemmRowB = kGemmBK * 2;   // bytes of one tile row in LDS: 8 chunks of 16 bytes

struct GemmParams {
  const unsigned char* x;   // bf16 [m, k]
  const unsigned char* w;   // bf16 [n, k]
  uint16_t* y;              // bf16 [m, n]
  float* part;              // fp32 [ksplit, m, n] when ksplit > 1
  int m, n, k, kchunk, ksplit;
  int mt, nt;               // tiles along m and n
  int per_xcd;              // tiles (of mt * nt * ksplit) each of the 8 XCD classes takes
};

// Tile of the workgroup.  Workgroups are dealt round-robin over the 8 XCDs
// (each with its own L2), so class c = id % 8 takes the c-th contiguous run
// of a tile order that walks kGemmGroupM m-tiles across every n-tile before
// the next group: the workgroups that run together on one XCD then share
// their x and W slices through its L2.  Returns false past the last tile.
constexpr int kGemmGroupM = 4;
__device__ __forceinline__ bool gemm_tile(const GemmParams& p, int& mt, int& nt, int& kz) {
  const int id = blockIdx.x;
  const int t = (id & 7) * p.per_xcd + (id >> 3);
  const int total = p.mt * p.nt * p.ksplit;
  if ((id >> 3) >= p.per_xcd || t >= total) return false;
  kz = t / (p.mt * p.nt);
  const int r = t - kz * (p.mt * p.nt);
  const int gsz = kGemmGroupM * p.nt;
  const int g = r / gsz;
  const int gm = min(kGemmGroupM, p.mt - g * kGemmGroupM);   // m-tiles in this group
  const int q = r - g * gsz;
  mt = g * kGemmGroupM + q % gm;
  nt = q / gm;
  return true;
}

// The 16-byte chunk c of tile row r sits at physical chunk c ^ ((r / 2) % 8).
// An MFMA operand read takes 32 consecutive rows at one logical chunk; in each
// group of 16 lanes the rows then cover all 64 banks once.
__device__ __forceinline__ int gemm_swz(int r) { return (r >> 1) & 7; }

template <int BM, int BN, int NW>
struct GemmShape {
  static constexpr int WAVES_M = BM >= 128 ? 2 : 1;      // the NW waves as WAVES_M x WAVES_N
  static constexpr int WAVES_N = NW / WAVES_M;
  static constexpr int WM = BM / (32 * WAVES_M);         // 32-row blocks per wave
  static constexpr int WN = BN / (32 * WAVES_N);         // 32-column blocks per wave
  static constexpr int A_BYTES = BM * kGemmRowB;
  static constexpr int STAGE = A_BYTES + BN * kGemmRowB;
  static constexpr int A_LOADS = A_BYTES / 1024;         // one wave-wide DMA instruction moves 1 KB (8 rows)
  static constexpr int B_LOADS = BN * kGemmRowB / 1024;
  static constexpr int LPW = (A_LOADS + B_LOADS) / NW;   // DMA instructions per wave per stage
  static_assert(WM >= 1 && WN >= 1 && (A_LOADS + B_LOADS) % NW == 0, "tile shape");
};

// STREAM_W: W tiles go with the non-temporal hint, for shapes with a single
// m-tile (each W byte is then read once; with several m-tiles the tiles of W
// are shared through L2 and stay cached).
template <int BM, int BN, int S, bool STREAM_W, int NW = 4>
__global__ __launch_bounds__(64 * NW) void verify_gemm(GemmParams p) {
  using SH = GemmShape<BM, BN, NW>;
  static_assert(S >= 2 && S <= 4 && (S - 2) * SH::LPW < 64, "ring depth");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S * SH::STAGE];
  const unsigned lds_base = (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / SH::WAVES_N, wn = wave % SH::WAVES_N;
  const int r32 = lane & 31, hh = lane >> 5;
  int mt, nt, kz;
  if (!gemm_tile(p, mt, nt, kz)) return;
  const int m0 = mt * BM;
  const int n0 = nt * BN;
  const int kb0 = kz * p.kchunk;
  const int kb1 = min(p.k, kb0 + p.kchunk);
  const int nst = (kb1 - kb0) / kGemmBK;
  const size_t rowg = (size_t)p.k * 2;   // bytes of one row of x or W

  // DMA slots of this wave: instruction j (= wave + NW i) fills rows 8j'..8j'+7
  // of the A tile (j < A_LOADS) or of the B tile; lane l takes row 8j' + l/8
  // and physical chunk l % 8, i.e. logical chunk (l % 8) ^ swz(row).
  unsigned src[SH::LPW], dst[SH::LPW];
  bool isb[SH::LPW];
#pragma unroll
  for (int i = 0; i < SH::LPW; ++i) {
    const int j = wave + NW * i;
    isb[i] = j >= SH::A_LOADS;
    const int jr = isb[i] ? j - SH::A_LOADS : j;
    const int row = 8 * jr + lane / 8;
    const int lc = (lane & 7) ^ gemm_swz(row);
    // rows past the matrix read its last row (their products are never stored)
    const int grow = isb[i] ? min(n0 + row, p.n - 1) - n0 : min(m0 + row, p.m - 1) - m0;
    src[i] = (unsigned)((size_t)grow * rowg + lc * 16);
    dst[i] = (unsigned)((isb[i] ? SH::A_BYTES : 0) + 8 * jr * kGemmRowB);
  }
  const unsigned char* xt = p.x + (size_t)m0 * rowg;
  const unsigned char* wt = p.w + (size_t)n0 * rowg;
  auto issue = [&](int st, int slot) {
    const size_t kofs = (size_t)(kb0 + st * kGemmBK) * 2;
#pragma unroll
    for (int i = 0; i < SH::LPW; ++i)
      if (isb[i]) dma16<STREAM_W>(wt + kofs, src[i], lds_base + (unsigned)(slot * SH::STAGE) + dst[i]);
      else dma16<false>(xt + kofs, src[i], lds_base + (unsigned)(slot * SH::STAGE) + dst[i]);
  };

  // operand offsets: lane reads row r32 of a 32-row block at logical chunk 2ks + hh
  int opoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) opoff[ks] = r32 * kGemmRowB + (((2 * ks + hh) ^ gemm_swz(r32)) * 16);

  f32x16 acc[SH::WM][SH::WN];
#pragma unroll
  for (int i = 0; i < SH::WM; ++i)
#pragma unroll
    for (int j = 0; j < SH::WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < nst) issue(st, st);
  for (int st = 0; st < nst; ++st) {
    // stage st has landed when at most the later stages already issued are in flight
    const int later = min(nst - st - 1, S - 2);
    if (later >= S - 2) wait_vmem<(S - 2) * SH::LPW>();
    else if (later >= 1) wait_vmem<SH::LPW>();
    else wait_vmem<0>();
    block_sync();
    if (st + S - 1 < nst) issue(st + S - 1, (st + S - 1) % S);
    const unsigned char* base = smem + (st % S) * SH::STAGE;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[SH::WM], b[SH::WN];
#pragma unroll
      for (int i = 0; i < SH::WM; ++i)
        a[i] = *(const bf16x8*)(base + (wm * SH::WM + i) * 32 * kGemmRowB + opoff[ks]);
#pragma unroll
      for (int j = 0; j < SH::WN; ++j)
        b[j] = *(const bf16x8*)(base + SH::A_BYTES + (wn * SH::WN + j) * 32 * kGemmRowB + opoff[ks]);
#pragma unroll
      for (int i = 0; i < SH::WM; ++i)
#pragma unroll
        for (int j = 0; j < SH::WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // D layout: lane l, entry e -> column l % 32, row (e/4)*8 + (l/32)*4 + e%4 of the block
#pragma unroll
  for (int i = 0; i < SH::WM; ++i)
#pragma unroll
    for (int j = 0; j < SH::WN; ++j) {
      const int n = n0 + (wn * SH::WN + j) * 32 + r32;
      if (n >= p.n) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + (wm * SH::WM + i) * 32 + (e >> 2) * 8 + hh * 4 + (e & 3);
        if (m >= p.m) continue;
        if (p.ksplit == 1) {
          const __bf16 v = (__bf16)acc[i][j][e];
          p.y[(size_t)m * p.n + n] = __builtin_bit_cast(uint16_t, v);
        } else {
          p.part[((size_t)kz * p.m + m) * p.n + n] = acc[i][j][e];
        }
      }
    }
}

// y = bf16(sum over splits, in split order, of the fp32 partials); 4 columns per thread.
// The partials come from other XCDs' L2 writebacks, so each load waits a full
// memory round trip: they are issued 8 at a time, then added in split order.
constexpr int kReduceBatch = 8;
__global__ __launch_bounds__(256) void verify_gemm_reduce(GemmParams p) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;   // index of a 4-column group
  const size_t total = (size_t)p.m * p.n / 4;
  if (q >= total) return;
  const size_t mn = (size_t)p.m * p.n;
  const float* src = p.part + q * 4;
  f32x4 s = *(const f32x4*)src;
  for (int z0 = 1; z0 < p.ksplit; z0 += kReduceBatch) {
    f32x4 v[kReduceBatch];
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j)
      v[j] = z0 + j < p.ksplit ? *(const f32x4*)(src + (size_t)(z0 + j) * mn) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j)
      if (z0 + j < p.ksplit) s += v[j];
  }
  const bf16x4 t = {(__bf16)s[0], (__bf16)s[1], (__bf16)s[2], (__bf16)s[3]};
  *(u32x2*)(p.y + q * 4) = __builtin_bit_cast(u32x2, t);
}

struct GemmPlan {
  int bm, bn, ksplit, kchunk;
};

// Tile by M (256 x 256 or 128 x 256 when that still gives three or two rounds of workgroups); K
// split so that small M still fills about two workgroups per CU in one round,
// as long as the fp32 partials (written and read once) stay below the bytes
// of W.
static GemmPlan gemm_plan(int m, int n, int k, int cus) {
  GemmPlan g;
  // 256 x 256 (the most flops per byte of ring fill) when it gives at least three whole rounds
  if (n % 256 == 0 && (long long)((m + 255) / 256) * (n / 256) >= 3LL * cus) {
    g.bm = g.bn = 256;
    g.ksplit = 1;
    g.kchunk = k;
    return g;
  }
  g.bm = m <= 32 ? 32 : m <= 256 ? 64 : 128;
  g.bn = (g.bm == 128 && n % 256 == 0 && (long long)((m + 127) / 128) * (n / 256) >= 2LL * cus) ? 256 : 128;
  const long long tiles = (long long)((m + g.bm - 1) / g.bm) * (n / g.bn);
  const long long target = (long long)cus * (g.bm == 128 ? 1 : 2);
  const int kblocks = k / kGemmBK;
  long long ks = target / std::max(1LL, tiles);
  ks = std::min<long long>(ks, std::max(1, kblocks / 4));
  ks = std::min<long long>(ks, std::max<long long>(1, (long long)k / (4LL * std::max(1, m))));
  ks = std::max<long long>(1, ks);
  const int per = (int)((kblocks + ks - 1) / ks);
  g.kchunk = per * kGemmBK;
  g.ksplit = (kblocks + per - 1) / per;
  return g;
}

}  // namespace sdv

using namespace sdv;

size_t sdv_gemm_workspace_bytes(int m, int n, int k) {
  const GemmPlan g = gemm_plan(m, n, k, 256);
  return g.ksplit > 1 ? (size_t)g.ksplit * m * n * sizeof(float) : 0;
}

hipError_t sdv_gemm_launch(const SdGemmLaunch& a) {
  int dev = 0, cus = 256;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  GemmPlan g = gemm_plan(a.m, a.n, a.k, std::min(cus, 256));
  if (g.ksplit > 1 && (size_t)g.ksplit * a.m * a.n * sizeof(float) > a.workspace_bytes) {
    // the workspace was sized for the largest CU count: fewer CUs never need more splits
    return hipErrorInvalidValue;
  }
  GemmParams p;
  p.x = (const unsigned char*)a.x;
  p.w = (const unsigned char*)a.w;
  p.y = (uint16_t*)a.y;
  p.part = (float*)a.workspace;
  p.m = a.m;
  p.n = a.n;
  p.k = a.k;
  p.kchunk = g.kchunk;
  p.ksplit = g.ksplit;
  p.mt = (a.m + g.bm - 1) / g.bm;
  p.nt = a.n / g.bn;
  const long long tiles = (long long)p.mt * p.nt * g.ksplit;
  p.per_xcd = (int)((tiles + 7) / 8);
  const dim3 grid((unsigned)(8LL * p.per_xcd));
  const bool stream_w = p.mt == 1;
  if (g.bm == 32 && stream_w) verify_gemm<32, 128, 4, true><<<grid, 256, 0, a.stream>>>(p);
  else if (g.bm == 32) verify_gemm<32, 128, 4, false><<<grid, 256, 0, a.stream>>>(p);
  else if (g.bm == 64 && stream_w) verify_gemm<64, 128, 3, true><<<grid, 256, 0, a.stream>>>(p);
  else if (g.bm == 64) verify_gemm<64, 128, 3, false><<<grid, 256, 0, a.stream>>>(p);
  else if (g.bm == 256) verify_gemm<256, 256, 2, false, 8><<<grid, 512, 0, a.stream>>>(p);
  else if (g.bn == 128) verify_gemm<128, 128, 4, false, 8><<<grid, 512, 0, a.stream>>>(p);
  else verify_gemm<128, 256, 3, false, 8><<<grid, 512, 0, a.stream>>>(p);
  if (g.ksplit > 1) {
    const size_t groups = (size_t)a.m * a.n / 4;
    verify_gemm_reduce<<<(unsigned)((groups + 255) / 256), 256, 0, a.stream>>>(p);
  }
  return hipGetLastError();
}
