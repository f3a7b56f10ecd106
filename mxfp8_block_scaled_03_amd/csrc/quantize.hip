// quantize.hip -- MX block quantization (mx_quantize) for gfx950.
//
// "Low-Precision GPU Programming", "Microscaling: the two-row experiment": per 32-element
// block along K take amax, choose the power-of-two scale S = 2^e that rounds amax/fmax
// upward (e >= -127; zero block -> S = 1), store e + 127 as the E8M0 byte and the codes
// RNE(x / S).  "Scale ownership and the GEMM dataflow": a partial final block is
// zero-padded.  "Scaling architectures" / "Current scaling": the amax reduction and the
// dependent cast stay on the device -- here in one pass over the data, since the MX amax
// is local to a block of 32 values.
//
// Encoding: v_cvt_scalef32_pk_{fp8,bf8}_{bf16,f32} computes RNE(x / scale) for a
// power-of-two fp32 scale; it is used for every block whose scale byte is 1..254 (the
// scale rule keeps |x / S| <= fmax, so its non-saturating overflow behaviour is never
// reached).  Scale byte 0 (S = 2^-127, not a normal fp32) takes the software encoder.
#include <type_traits>

#include "codec.hpp"
#include "internal.hpp"
#include "mxblock.hpp"

namespace mxq {
namespace {

constexpr int kThreads = 256;
using namespace mxblock;

// Load chunk: elements k0 .. k0+7 of a line starting at `line` (element pointer).
template <int SRC_BF16, bool VEC>
__device__ __forceinline__ void load_chunk(Chunk<SRC_BF16>& c, const void* line, int64_t k0, int64_t K) {
  if (VEC) {
    if (k0 < K) {
      if (SRC_BF16) {
        uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(line) + k0);
        c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(line) + k0);
        uint4 v0 = p[0], v1 = p[1];
        c.w[0] = v0.x; c.w[1] = v0.y; c.w[2] = v0.z; c.w[3] = v0.w;
        c.w[4] = v1.x; c.w[5] = v1.y; c.w[6] = v1.z; c.w[7] = v1.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < (SRC_BF16 ? 4 : 8); ++i) c.w[i] = 0u;
    }
  } else {
    if (SRC_BF16) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(line);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo = (k0 + 2 * i < K) ? p[k0 + 2 * i] : 0u;
        uint32_t hi = (k0 + 2 * i + 1 < K) ? p[k0 + 2 * i + 1] : 0u;
        c.w[i] = lo | (hi << 16);
      }
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(line);
#pragma unroll
      for (int i = 0; i < 8; ++i) c.w[i] = (k0 + i < K) ? p[k0 + i] : 0u;
    }
  }
}

// One lane per 32-element block: the lane loads the block's 64 (bf16) or 128 (fp32) bytes
// with 16-byte loads, reduces the amax in registers, encodes with 16 two-value
// conversions and stores 32 code bytes with two 16-byte stores; a wave covers 64
// consecutive blocks, so its 64 scale bytes form one contiguous run.  Blocks are
// numbered g = row * nb + b (FLAT problems are one dense run: row 0, b = g).  One block
// per thread and a large grid keep enough loads in flight to stream HBM.
template <int SRC_BF16, int F, bool FLAT, bool VEC, int R>
__global__ __launch_bounds__(kThreads) void k_quant_rows(const void* __restrict__ src, int64_t ld_src, int64_t K,
                                                        int64_t nb, int64_t nblocks, uint8_t* __restrict__ codes,
                                                        int64_t ld_codes, uint8_t* __restrict__ scales, int64_t ld_scales) {
  constexpr int ES = SRC_BF16 ? 2 : 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < nblocks; g += stride) {
    const int64_t row = FLAT ? 0 : g / nb;
    const int64_t b = FLAT ? g : g - row * nb;
    const char* line = reinterpret_cast<const char*>(src) + row * ld_src * ES;
    Chunk<SRC_BF16> c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      load_chunk<SRC_BF16, VEC>(c[q], line, 32 * b + 8 * q, FLAT ? (int64_t)INT64_MAX : K);
    uint32_t amax = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = chunk_abs_max<SRC_BF16>(c[q]);
      amax = amax > a ? amax : a;
    }
    const uint32_t sb = scale_byte_rule<F, R>(amax);
    uint32_t d[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) encode_chunk<SRC_BF16, F, R>(c[q], sb, d[2 * q], d[2 * q + 1]);
    uint4* out = reinterpret_cast<uint4*>(codes + row * ld_codes + 32 * b);
    out[0] = make_uint4(d[0], d[1], d[2], d[3]);
    out[1] = make_uint4(d[4], d[5], d[6], d[7]);
    scales[row * ld_scales + b] = (uint8_t)sb;
  }
}

// Columnwise, straight from HBM: the path for sources whose rows are not whole, aligned
// 16-byte pieces (k_quant_cols_lds below takes the rest).  A wave's task is 512 rows (16
// blocks, taken as 4 sub-tiles of 128 rows) of 64 consecutive columns, one column per
// lane: every load of
// the wave reads one contiguous row segment (128 bytes of bf16, 256 of fp32).  The lane
// reduces and encodes its column a block at a time, keeps the sub-tile's 128 codes in
// registers and writes them as one burst of eight 16-byte stores; the task's 16 scale
// bytes go out as one 16-byte store at the end.  No LDS and no barrier.
// Counter evidence behind the shape (2^28 bf16, WRITE_SIZE against the 264 MiB the
// kernel writes): a column's 128-byte line of codes written in 32-byte pieces, whether by
// four waves or by one wave a block apart, gave 380-415 MiB; scale bytes written 4 at a
// time from tiles on different XCDs gave 340 MiB with whole code lines; whole code lines
// and 16-byte scale pieces whose 128-byte line is completed on one XCD give 286 MiB.
// The 4 waves of a workgroup take 4 adjacent column strips of one 512-row group;
// workgroup tasks are numbered strip-major (the groups of one strip consecutive, so the 8
// tasks that share a column's 128-byte scale line run together on one XCD) and dealt to
// the XCDs in contiguous chunks (workgroup g runs on XCD g % 8).
constexpr int kColGroupRows = 512;   // rows of a task: 16 blocks
constexpr int kXcds = 8;
constexpr int kColStrip = 64;        // columns per wave task

// gx column strips and ng = ceil(rows / 512) row groups; workgroup tasks (4 strips x 1
// group) number wg_total = ceil(gx / 4) * ng; XCD g % 8 owns tasks
// [xcd * per_xcd, (xcd + 1) * per_xcd) and its workgroups stride through them by
// slots = gridDim / 8.
struct ColTiles {
  int64_t wg_total, per_xcd, gx, ng;
};

// BUF: the task's rows are read through a buffer descriptor based at the task's first
// element of row r0 whose range ends at the last valid element, so rows past the matrix
// read as zero (the zero padding) and each load is one scalar row offset plus the lane's
// byte offset; it needs 512 rows within 2^31 bytes, otherwise element loads with explicit
// bounds.  A bf16 value lands in the low half of its dword.  vsc: scales and ld_scales
// are 16-byte aligned, so a whole task's 16 scale bytes are one store.
template <int SRC_BF16, int F, bool BUF, int R>
__global__ __launch_bounds__(kThreads) void k_quant_cols(const void* __restrict__ src, int64_t rows, int64_t cols,
                                                        int64_t ld_src, int64_t nb, uint8_t* __restrict__ codes,
                                                        int64_t ld_codes, uint8_t* __restrict__ scales,
                                                        int64_t ld_scales, ColTiles tiles, int vsc) {
  constexpr int ES = SRC_BF16 ? 2 : 4;
  const int64_t xcd = blockIdx.x % kXcds;
  const int64_t slots = gridDim.x / kXcds;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // the wave index: scalar
  for (int64_t s = blockIdx.x / kXcds; s < tiles.per_xcd; s += slots) {
    const int64_t t = xcd * tiles.per_xcd + s;
    if (t >= tiles.wg_total) break;
    const int64_t xw = t / tiles.ng, g = t - xw * tiles.ng;
    const int64_t x = 4 * xw + wv;
    if (x >= tiles.gx) continue;                   // uniform over the wave
    const int64_t c0 = x * kColStrip, col = c0 + lane;
    const bool live = col < cols;
    const int64_t b0 = 16 * g, r0 = 32 * b0;
    const int nblk = nb - b0 < 16 ? (int)(nb - b0) : 16;          // uniform
    const bool full = vsc && nblk == 16;
    // (unused without BUF: a descriptor of range 0)
    const int64_t nvalid = rows - r0 < kColGroupRows ? rows - r0 : kColGroupRows;
    const char* base = reinterpret_cast<const char*>(src) + (BUF ? (r0 * ld_src + c0) * ES : 0);
    const uint32_t range = BUF ? (uint32_t)(((nvalid - 1) * ld_src + (cols - c0)) * ES) : 0u;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)range, 0x00020000);
    const int row_bytes = BUF ? (int)(ld_src * ES) : 0;
    uint32_t q[4];                                 // scale bytes of the task, block k in byte k
    for (int st = 0; st < 4; ++st) {
      const int kb0 = 4 * st;
      if (kb0 >= nblk) break;                      // uniform
      const int nsub = nblk - kb0 < 4 ? nblk - kb0 : 4;
      uint32_t c[32];                              // codes of the sub-tile's (up to) 4 blocks
      uint32_t sw = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j >= nsub) break;                      // uniform
        const int k = kb0 + j;
        uint32_t w[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (BUF) {
            w[i] = SRC_BF16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, 2 * lane, (32 * k + i) * row_bytes, 0)
                            : __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lane, (32 * k + i) * row_bytes, 0);
          } else {
            const int64_t r = r0 + 32 * k + i;
            w[i] = 0u;
            if (live && r < rows)
              w[i] = SRC_BF16 ? (uint32_t)reinterpret_cast<const uint16_t*>(src)[r * ld_src + col]
                              : reinterpret_cast<const uint32_t*>(src)[r * ld_src + col];
          }
        }
        uint32_t sb;
        if (SRC_BF16) {
          uint32_t m = 0;
#pragma unroll
          for (int i = 0; i < 32; ++i) m = pk_abs_max_bf16(m, w[i]);
          sb = scale_byte_rule<F, R>(m << 16);
          encode_block32_bf16_half<F, R>(w, false, sb, &c[8 * j]);
        } else {
          uint32_t amax = 0;
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const uint32_t a = w[i] & 0x7FFFFFFFu;
            amax = amax > a ? amax : a;
          }
          sb = scale_byte_rule<F, R>(amax);
          encode_block32<F, R>(w, sb, &c[8 * j]);
        }
        sw |= sb << (8 * j);
      }
      q[st] = sw;
      if (!live) continue;
      uint4* dst = reinterpret_cast<uint4*>(codes + col * ld_codes + 32 * (b0 + kb0));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j >= nsub) break;
        dst[2 * j] = make_uint4(c[8 * j], c[8 * j + 1], c[8 * j + 2], c[8 * j + 3]);
        dst[2 * j + 1] = make_uint4(c[8 * j + 4], c[8 * j + 5], c[8 * j + 6], c[8 * j + 7]);
      }
      if (!full)
        for (int j = 0; j < nsub; ++j) scales[col * ld_scales + b0 + kb0 + j] = (uint8_t)(sw >> (8 * j));
    }
    if (full && live) *reinterpret_cast<uint4*>(scales + col * ld_scales + b0) = make_uint4(q[0], q[1], q[2], q[3]);
  }
}

// Columnwise through LDS, for rows of whole 16-byte pieces (bf16: cols % 8 == 0,
// fp32: cols % 4 == 0; 16-byte aligned src and row pitch).  A workgroup takes one tile of
// 128 rows (4 blocks) x 64 columns (16 KB of bf16, 32 KB of fp32), so a launch has many
// small independent workgroups.  The tile moves from HBM with 16-byte loads (a wave load
// covers whole 128/256-byte row segments), is written to LDS row-major and read back down
// the columns: lane 4c + kb of wave w takes column 16w + c, block kb.  Row r is stored
// with its dword index xor SWZ * ((r >> 5) & 3) (SWZ = the dwords of 8 columns), so the
// four blocks read by a half-wave fall on different banks.  The four lanes of a column
// write its 128-byte line of codes in the same pair of store instructions.
// Earlier shapes of this kernel, on 2^28 bf16: the same tile without the swizzle (4-way
// LDS bank conflicts, 20% of the cycles) took 204 us; a direct kernel with one column per
// lane and one 128/256-byte row segment per load took 240 us (its loads touch one cache
// line each: the texture address unit stalled on the L1 3x as often as the rowwise
// kernel's at the same L2 latency); a persistent kernel with 128 x 128 tiles, 3
// workgroups per CU and a register prefetch took 221 us.
// Tile t of a gy x gx grid of tiles, in groups of GH x GW tiles: x fastest inside a
// group, groups in row-band order, narrower or shorter groups at the right and bottom
// edges (a bijection of [0, gx * gy)).  Workgroup g takes tile (g % 8) * ceil(n / 8) + g / 8,
// so each XCD runs a contiguous run of groups.  For the transposing kernels the group
// shape trades the two halves of the traffic: the workgroups in flight on an XCD read
// GW adjacent 128-byte pieces of each source row (long DRAM runs) and write the
// transposed codes at GH different row offsets (spread over the memory channels; a
// whole row band at one offset, the plain row-major order, writes every line at the same
// offset within its 16 KB row).  Measured on 2^28 bf16 columnwise: row-major order
// 198 us; 16 x 16 groups 169 us; 8 x 32 159 us; 8 x 64 156 us; 2 x 128 175 us;
// 64 x 4 188 us.
template <int64_t GH, int64_t GW>
__device__ __forceinline__ void grouped_tile(int64_t t, int64_t gx, int64_t gy, int64_t& y, int64_t& x) {
  const int64_t band = t / (GH * gx), rem = t - band * GH * gx;
  const int64_t hb = gy - GH * band < GH ? gy - GH * band : GH;
  const int64_t grp = rem / (GW * hb), r2 = rem - grp * GW * hb;
  const int64_t wdt = gx - GW * grp < GW ? gx - GW * grp : GW;
  y = GH * band + r2 / wdt;
  x = GW * grp + r2 % wdt;
}

constexpr int kColGroupH = 8, kColGroupW = 64;    // columnwise tile group: rows x columns of tiles

template <int SRC_BF16>
struct CtGeom {
  static constexpr int ES = SRC_BF16 ? 2 : 4;
  static constexpr int TC = 64;                     // tile columns (4 lanes each)
  static constexpr int RW = TC * ES / 4;            // dwords per tile row: 32 / 64
  static constexpr int PPR = TC * ES / 16;          // 16-byte pieces per row: 8 / 16
  static constexpr int NP = 128 * PPR / kThreads;   // pieces per thread: 4 / 8
  static constexpr int CPW = TC / 4;                // columns per wave: 16
  static constexpr int SWZ = 2 * ES;                // dwords of a half-wave's 8 columns
};

// SR: stochastically rounded codes (encode_sr with the block's Philox words, line col,
// block b -> block index col * nb + b, as k_quant_cols_sr) under the RNE quantizer's scale.
template <int SRC_BF16, int F, int R, bool SR>
__global__ __launch_bounds__(kThreads) void k_quant_cols_lds(const void* __restrict__ src, int64_t rows,
                                                            int64_t cols, int64_t ld_src, int64_t nb,
                                                            uint8_t* __restrict__ codes, int64_t ld_codes,
                                                            uint8_t* __restrict__ scales, int64_t ld_scales,
                                                            int64_t gx, int64_t ntiles, int64_t per_xcd,
                                                            uint64_t seed) {
  typedef CtGeom<SRC_BF16> G;
  __shared__ __align__(16) uint32_t ctile[128 * G::RW];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t t = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (t >= ntiles) return;                           // the whole workgroup, before any barrier
  int64_t y, x;
  grouped_tile<kColGroupH, kColGroupW>(t, gx, ntiles / gx, y, x);
  const int64_t c0 = x * G::TC, r0 = 128 * y;
  const int64_t nvalid = rows - r0 < 128 ? rows - r0 : 128;
  const char* base = reinterpret_cast<const char*>(src) + (r0 * ld_src + c0) * G::ES;
  const uint32_t range = (uint32_t)(((nvalid - 1) * ld_src + (cols - c0)) * G::ES);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)range, 0x00020000);
  const int row_bytes = (int)(ld_src * G::ES);
  uint4 v[G::NP];
#pragma unroll
  for (int q = 0; q < G::NP; ++q) {
    const int p = tid + kThreads * q;
    const auto d = __builtin_amdgcn_raw_buffer_load_b128(rs, (p / G::PPR) * row_bytes + (p % G::PPR) * 16, 0, 0);
    v[q] = make_uint4((uint32_t)d[0], (uint32_t)d[1], (uint32_t)d[2], (uint32_t)d[3]);
  }
#pragma unroll
  for (int q = 0; q < G::NP; ++q) {
    const int p = tid + kThreads * q;
    const int row = p / G::PPR;
    const int d = ((p % G::PPR) * 4) ^ (G::SWZ * ((row >> 5) & 3));
    *reinterpret_cast<uint4*>(&ctile[row * G::RW + d]) = v[q];
  }
  __syncthreads();
  const int kb = lane & 3;
  const int cl = G::CPW * wv + (lane >> 2);          // column within the tile
  const int64_t col = c0 + cl, b = 4 * y + kb;
  if (col >= cols || b >= nb) return;                // no barrier follows
  uint32_t w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int row = 32 * kb + i;
    const int sw = G::SWZ * kb;                      // (row >> 5) & 3 == kb
    if (SRC_BF16) {
      const int d = (cl >> 1) ^ sw;
      w[i] = (uint32_t)reinterpret_cast<const uint16_t*>(ctile)[2 * (row * G::RW + d) + (cl & 1)];
    } else {
      w[i] = ctile[row * G::RW + (cl ^ sw)];
    }
  }
  uint32_t c[8], sb;
  if (SRC_BF16) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = pk_abs_max_bf16(m, w[i]);
    sb = scale_byte_rule<F, R>(m << 16);
    if (!SR) encode_block32_bf16_half<F, R>(w, false, sb, c);
  } else {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t a = w[i] & 0x7FFFFFFFu;
      amax = amax > a ? amax : a;
    }
    sb = scale_byte_rule<F, R>(amax);
    if (!SR) encode_block32<F, R>(w, sb, c);
  }
  if (SR) {
    if (sb == 255u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = 0x7F7F7F7Fu;
    } else {
      uint32_t rnd[32];
      block_random24((uint64_t)col * (uint64_t)nb + (uint64_t)b, seed, rnd);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t cw = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t vb = SRC_BF16 ? w[4 * i + j] << 16 : w[4 * i + j];
          cw |= encode_sr<F>(vb, sb, rnd[4 * i + j]) << (8 * j);
        }
        c[i] = cw;
      }
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + col * ld_codes + 32 * b);
  dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
  dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
  scales[col * ld_scales + b] = (uint8_t)sb;
}

// Column tasks of a [rows][cols] problem and the launch size: 8 * ceil(tasks / 8)
// workgroups, capped so that each XCD's workgroups loop (every wave reaches the end of
// the loop: the trip count depends only on the workgroup index and the task count).
static ColTiles col_tiles(int64_t rows, int64_t cols, int64_t* grid) {
  ColTiles t;
  t.gx = (cols + kColStrip - 1) / kColStrip;
  t.ng = (rows + kColGroupRows - 1) / kColGroupRows;
  t.wg_total = (t.gx + 3) / 4 * t.ng;
  t.per_xcd = (t.wg_total + kXcds - 1) / kXcds;
  const int64_t cap = (int64_t)device_cu_count() * 8 / kXcds;    // workgroups per XCD
  *grid = kXcds * (t.per_xcd < cap ? t.per_xcd : cap);
  return t;
}

// The LDS-staged column kernels (dual, stochastic rounding, caller-owned scales) take
// tiles of 128 rows x 64 columns.
constexpr int kColTileRows = 128;
constexpr int kColTileCols = 64;


// Both orientations from one read ("Microscaling: the two-row experiment", last
// paragraph: regrouping from 1x32 to 32x1 changes which values share a scale, so the
// columnwise codes are derived from the wide data, not from the rowwise bytes).  A
// workgroup takes a tile of 128 rows x 64 columns: thread t loads chunks (8 values) of
// rows t/8 + 32k, chunk t%8, and the four lanes holding one 32-value row block reduce it
// with DPP and write its rowwise codes and scale straight from registers; the tile also
// goes to LDS, from which the columnwise blocks are encoded exactly as in k_quant_cols.
template <int SRC_BF16, int F, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_dual(const void* __restrict__ src, int64_t rows, int64_t cols,
                                                        int64_t ld_src, uint8_t* __restrict__ rcodes, int64_t ld_rc,
                                                        uint8_t* __restrict__ rscales, int64_t ld_rs,
                                                        uint8_t* __restrict__ ccodes, int64_t ld_cc,
                                                        uint8_t* __restrict__ cscales, int64_t ld_cs) {
  typedef typename std::conditional<SRC_BF16, uint16_t, uint32_t>::type E;
  constexpr int ES = (int)sizeof(E);
  constexpr int PW = kColTileCols * ES / 4 + 1;      // LDS row pitch in dwords
  __shared__ uint32_t tile[kColTileRows * PW];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kColTileCols;
  const int64_t nb_r = (cols + 31) / 32, nb_c = (rows + 31) / 32;
  const int64_t kp_r = 32 * nb_r;
  const int tq = tid & 7;                             // chunk within the tile row
  for (int64_t ty = blockIdx.y; ty * kColTileRows < rows; ty += gridDim.y) {
    const int64_t r0 = ty * kColTileRows;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int tr = (tid >> 3) + 32 * k;
      const int64_t r = r0 + tr;
      const int64_t cc = c0 + 8 * tq;
      Chunk<SRC_BF16> ch;
      if (r < rows) {
        const char* line = reinterpret_cast<const char*>(src) + r * ld_src * ES;
        load_chunk<SRC_BF16, VEC>(ch, line, cc, cols);
      } else {
#pragma unroll
        for (int i = 0; i < (SRC_BF16 ? 4 : 8); ++i) ch.w[i] = 0u;
      }
      // tile copy for the columnwise pass
      uint32_t* dst = &tile[tr * PW + 8 * tq * ES / 4];
#pragma unroll
      for (int i = 0; i < (SRC_BF16 ? 4 : 8); ++i) dst[i] = ch.w[i];
      // rowwise block of this quad (every lane of the wave takes part in the DPP)
      const uint32_t amax = quad_max(chunk_abs_max<SRC_BF16>(ch));
      const uint32_t sb = scale_byte_from_amax<F>(amax);
      uint32_t d0, d1;
      encode_chunk<SRC_BF16, F>(ch, sb, d0, d1);
      if (r < rows && cc < kp_r) {
        *reinterpret_cast<uint2*>(rcodes + r * ld_rc + cc) = make_uint2(d0, d1);
        if ((tq & 3) == 0) rscales[r * ld_rs + (cc >> 5)] = (uint8_t)sb;
      }
    }
    __syncthreads();
    const int c = tid >> 2, kb = tid & 3;
    const int64_t col = c0 + c, b = r0 / 32 + kb;
    if (col < cols && b < nb_c) {
      uint32_t amax = 0;
      uint32_t v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int row = 32 * kb + i;
        uint32_t x;
        if (SRC_BF16) x = (uint32_t)reinterpret_cast<const uint16_t*>(tile)[row * PW * 2 + c] << 16;
        else x = tile[row * PW + c];
        v[i] = x;
        const uint32_t a = x & 0x7FFFFFFFu;
        amax = amax > a ? amax : a;
      }
      const uint32_t sb = scale_byte_from_amax<F>(amax);
      uint32_t out[8];
      encode_block32<F>(v, sb, out);
      uint4* dst = reinterpret_cast<uint4*>(ccodes + col * ld_cc + 32 * b);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      cscales[col * ld_cs + b] = (uint8_t)sb;
    }
    __syncthreads();
  }
}
// Both orientations through LDS, for rows of whole 16-byte pieces (the conditions of
// k_quant_cols_lds).  A workgroup takes one tile of 128 rows x 128 columns (32 KB of
// bf16, 64 KB of fp32): thread t's q-th chunk (8 values: one 16-byte load of bf16, two of
// fp32) is row p / 16, chunk p % 16 with p = t + 256 q, so the four lanes of a quad hold
// one 32-value row block (reduced with DPP) and the 16 lanes of a row write its 128-byte
// line of rowwise codes in one store instruction.  Columns past cols read as zero (they
// are the rowwise zero padding).  The tile goes to LDS in the swizzled layout of
// k_quant_cols_lds and is read back down the columns in two passes of 64 columns: lane
// 4c + kb of wave w takes column 64u + 16w + c, block kb, and the four lanes of a column
// write its 128-byte line of columnwise codes together.  With 128 x 64 tiles, the rowwise
// codes went out as 64-byte half-lines from two workgroups and the counters showed 17%
// more HBM write bytes than the kernel writes.
constexpr int kDualGroupH = 8, kDualGroupW = 32;  // dual tile group (tiles of 128 columns)

template <int SRC_BF16, int F>
__global__ __launch_bounds__(kThreads) void k_quant_dual_lds(const void* __restrict__ src, int64_t rows, int64_t cols,
                                                            int64_t ld_src, uint8_t* __restrict__ rcodes, int64_t ld_rc,
                                                            uint8_t* __restrict__ rscales, int64_t ld_rs,
                                                            uint8_t* __restrict__ ccodes, int64_t ld_cc,
                                                            uint8_t* __restrict__ cscales, int64_t ld_cs, int64_t gx,
                                                            int64_t ntiles, int64_t per_xcd) {
  constexpr int ES = SRC_BF16 ? 2 : 4;
  constexpr int RW = 128 * ES / 4;                 // dwords per tile row: 64 / 128
  constexpr int CW = 8 * ES / 4;                   // dwords per chunk: 4 / 8
  constexpr int SWZ = 2 * ES;                      // dwords of a half-wave's 8 columns
  extern __shared__ __align__(16) uint32_t dtile[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  // grouped tile order (grouped_tile), XCD chunks: the tiles that share a row's line of
  // rowwise scale bytes also run on one XCD
  const int64_t t = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (t >= ntiles) return;                           // the whole workgroup, before any barrier
  int64_t y, x;
  grouped_tile<kDualGroupH, kDualGroupW>(t, gx, ntiles / gx, y, x);
  const int64_t c0 = 128 * x, r0 = 128 * y;
  const int64_t nb_r = (cols + 31) / 32, nb_c = (rows + 31) / 32;
  const int64_t kp_r = 32 * nb_r;
  const int64_t nvalid = rows - r0 < 128 ? rows - r0 : 128;
  const char* base = reinterpret_cast<const char*>(src) + (r0 * ld_src + c0) * ES;
  const uint32_t range = (uint32_t)(((nvalid - 1) * ld_src + (cols - c0)) * ES);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)range, 0x00020000);
  const int row_bytes = (int)(ld_src * ES);
  const int chunk = tid & 15;
  const int64_t cc = c0 + 8 * chunk;               // first column of the lane's chunks
  // every load of the tile is issued before the first store: the compiler cannot move a
  // buffer load across the code stores, so loads interleaved with them would each wait a
  // full memory round trip in turn
  Chunk<SRC_BF16> chs[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = (tid >> 4) + 16 * q;
#pragma unroll
    for (int h = 0; h < ES / 2; ++h) {             // 16-byte pieces of the chunk
      const auto d = __builtin_amdgcn_raw_buffer_load_b128(rs, row * row_bytes + (8 * chunk) * ES + 16 * h, 0, 0);
      const bool in = cc + (16 / ES) * h < cols;   // pieces past cols are padding
#pragma unroll
      for (int i = 0; i < 4; ++i) chs[q].w[4 * h + i] = in ? (uint32_t)d[i] : 0u;
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = (tid >> 4) + 16 * q;
    const Chunk<SRC_BF16>& ch = chs[q];
    const int sw = SWZ * ((row >> 5) & 3);
#pragma unroll
    for (int h = 0; h < ES / 2; ++h)
      *reinterpret_cast<uint4*>(&dtile[row * RW + ((CW * chunk + 4 * h) ^ sw)]) =
          make_uint4(ch.w[4 * h], ch.w[4 * h + 1], ch.w[4 * h + 2], ch.w[4 * h + 3]);
    // rowwise block of this quad (every lane of the wave takes part in the DPP)
    const uint32_t amax = quad_max(chunk_abs_max<SRC_BF16>(ch));
    const uint32_t sb = scale_byte_from_amax<F>(amax);
    uint32_t d0, d1;
    encode_chunk<SRC_BF16, F>(ch, sb, d0, d1);
    const int64_t r = r0 + row;
    if (r < rows && cc < kp_r) {
      *reinterpret_cast<uint2*>(rcodes + r * ld_rc + cc) = make_uint2(d0, d1);
      if ((chunk & 3) == 0) rscales[r * ld_rs + (cc >> 5)] = (uint8_t)sb;
    }
  }
  __syncthreads();
  const int kb = lane & 3;
  const int64_t b = 4 * y + kb;
  if (b >= nb_c) return;                           // no barrier follows
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int cl = 64 * u + 16 * wv + (lane >> 2);
    const int64_t col = c0 + cl;
    if (col >= cols) break;
    uint32_t w[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int row = 32 * kb + i;
      const int sw = SWZ * kb;
      if (SRC_BF16) w[i] = (uint32_t)reinterpret_cast<const uint16_t*>(dtile)[2 * (row * RW + ((cl >> 1) ^ sw)) + (cl & 1)];
      else w[i] = dtile[row * RW + (cl ^ sw)];
    }
    uint32_t c[8], sb;
    if (SRC_BF16) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) m = pk_abs_max_bf16(m, w[i]);
      sb = scale_byte_from_amax<F>(m << 16);
      encode_block32_bf16_half<F>(w, false, sb, c);
    } else {
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t a = w[i] & 0x7FFFFFFFu;
        amax = amax > a ? amax : a;
      }
      sb = scale_byte_from_amax<F>(amax);
      encode_block32<F>(w, sb, c);
    }
    uint4* dst = reinterpret_cast<uint4*>(ccodes + col * ld_cc + 32 * b);
    dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
    dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
    cscales[col * ld_cs + b] = (uint8_t)sb;
  }
}

// Rowwise quantize with stochastically rounded codes: one lane per block as in
// k_quant_rows; the block's scale byte is the RNE quantizer's, its 32 codes are drawn by
// encode_sr with the block's Philox words (line l, block b -> block index l * nb + b).
template <int SRC_BF16, int F, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_rows_sr(const void* __restrict__ src, int64_t ld_src, int64_t K,
                                                           int64_t nb, int64_t nblocks, uint8_t* __restrict__ codes,
                                                           int64_t ld_codes, uint8_t* __restrict__ scales,
                                                           int64_t ld_scales, uint64_t seed) {
  constexpr int ES = SRC_BF16 ? 2 : 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < nblocks; g += stride) {
    const int64_t row = g / nb, b = g - row * nb;
    const char* line = reinterpret_cast<const char*>(src) + row * ld_src * ES;
    Chunk<SRC_BF16> c[4];
    uint32_t amax = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      load_chunk<SRC_BF16, VEC>(c[q], line, 32 * b + 8 * q, K);
      const uint32_t a = chunk_abs_max<SRC_BF16>(c[q]);
      amax = amax > a ? amax : a;
    }
    const uint32_t sb = scale_byte_from_amax<F>(amax);
    uint32_t d[8];
    if (sb == 255u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = 0x7F7F7F7Fu;
    } else {
      uint32_t r[32];
      block_random24((uint64_t)g, seed, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int el = 4 * i + j;
          w |= encode_sr<F>(value_bits<SRC_BF16>(c[el >> 3], el & 7), sb, r[el]) << (8 * j);
        }
        d[i] = w;
      }
    }
    uint4* out = reinterpret_cast<uint4*>(codes + row * ld_codes + 32 * b);
    out[0] = make_uint4(d[0], d[1], d[2], d[3]);
    out[1] = make_uint4(d[4], d[5], d[6], d[7]);
    scales[row * ld_scales + b] = (uint8_t)sb;
  }
}

// Columnwise quantize with stochastically rounded codes: the tile scheme of k_quant_cols;
// thread (column c, block kb) draws the Philox words of block index col * nb + b.
template <int SRC_BF16, int F, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_cols_sr(const void* __restrict__ src, int64_t rows, int64_t cols,
                                                           int64_t ld_src, int64_t nb, uint8_t* __restrict__ codes,
                                                           int64_t ld_codes, uint8_t* __restrict__ scales,
                                                           int64_t ld_scales, uint64_t seed) {
  typedef typename std::conditional<SRC_BF16, uint16_t, uint32_t>::type E;
  constexpr int PW = kColTileCols * (int)sizeof(E) / 4 + 1;
  __shared__ uint32_t tile[kColTileRows * PW];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kColTileCols;
  const E* s = reinterpret_cast<const E*>(src);
  for (int64_t ty = blockIdx.y; ty * kColTileRows < rows; ty += gridDim.y) {
    const int64_t r0 = ty * kColTileRows;
    constexpr int EPV = 16 / sizeof(E);
    constexpr int PPR = kColTileCols / EPV;
    for (int p = tid; p < kColTileRows * PPR; p += kThreads) {
      const int tr = p / PPR, tc = (p % PPR) * EPV;
      const int64_t r = r0 + tr, cc = c0 + tc;
      uint32_t* dst = &tile[tr * PW + tc * (int)sizeof(E) / 4];
      if (VEC && r < rows && cc + EPV <= cols) {
        const uint4 v = *reinterpret_cast<const uint4*>(s + r * ld_src + cc);
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
      } else {
        E e[EPV];
#pragma unroll
        for (int i = 0; i < EPV; ++i) e[i] = (r < rows && cc + i < cols) ? s[r * ld_src + cc + i] : (E)0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (SRC_BF16) dst[w] = (uint32_t)e[2 * w] | ((uint32_t)e[2 * w + 1] << 16);
          else dst[w] = (uint32_t)e[w];
        }
      }
    }
    __syncthreads();
    const int c = tid >> 2, kb = tid & 3;
    const int64_t col = c0 + c, b = r0 / 32 + kb;
    if (col < cols && b < nb) {
      uint32_t amax = 0;
      uint32_t v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int row = 32 * kb + i;
        uint32_t x;
        if (SRC_BF16) x = (uint32_t)reinterpret_cast<const uint16_t*>(tile)[row * PW * 2 + c] << 16;
        else x = tile[row * PW + c];
        v[i] = x;
        const uint32_t a = x & 0x7FFFFFFFu;
        amax = amax > a ? amax : a;
      }
      const uint32_t sb = scale_byte_from_amax<F>(amax);
      uint32_t out[8];
      if (sb == 255u) {
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = 0x7F7F7F7Fu;
      } else {
        uint32_t rnd[32];
        block_random24((uint64_t)col * (uint64_t)nb + (uint64_t)b, seed, rnd);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t w = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) w |= encode_sr<F>(v[4 * i + j], sb, rnd[4 * i + j]) << (8 * j);
          out[i] = w;
        }
      }
      uint4* dst = reinterpret_cast<uint4*>(codes + col * ld_codes + 32 * b);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      scales[col * ld_scales + b] = (uint8_t)sb;
    }
    __syncthreads();
  }
}
// Codes of one 32-value block under a caller-owned scale byte sb ("Worked failure: stale
// delayed scale"): RNE-satfinite(x / S) by the exact software encoder (x / S by ldexp,
// exact unless it over- or underflows fp32, where the code is fmax or zero anyway), NaN ->
// 0x7F, sb = 255 -> the whole block 0x7F.  Counts the elements saturated (|x / S| > fmax)
// and the nonzero ones that become a zero code; returns the block's abs-max bit pattern.
// n_real: elements of the block inside the line (the rest are padding, code 0x00).
template <int F>
__device__ __forceinline__ uint32_t encode_scaled_block(const uint32_t v[32], uint32_t sb, int n_real, uint32_t out[8],
                                                        uint32_t& nclip, uint32_t& nflush) {
  uint32_t amax = 0;
  nclip = nflush = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int el = 4 * i + j;
      const uint32_t x = v[el];
      const uint32_t mag = x & 0x7FFFFFFFu;
      uint32_t c = 0u;
      if (el < n_real) {
        amax = amax > mag ? amax : mag;
        if (sb == 255u || mag > 0x7F800000u) {
          c = 0x7Fu;
        } else {
          const float a = ldexpf(__uint_as_float(x), 127 - (int)sb);
          const bool clip = (__float_as_uint(a) & 0x7FFFFFFFu) > Fp8<F>::max_bits;
          c = encode_rne_sat<F>(a);
          nclip += clip ? 1u : 0u;
          nflush += (mag != 0u && (c & 0x7Fu) == 0u) ? 1u : 0u;
        }
      } else if (sb == 255u) {
        c = 0x7Fu;
      }
      w |= c << (8 * j);
    }
    out[i] = w;
  }
  return amax;
}

// Rowwise quantize with caller-owned scale bytes: one lane per block.
template <int SRC_BF16, int F, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_rows_scaled(
    const void* __restrict__ src, int64_t ld_src, int64_t K, int64_t nb, int64_t nblocks,
    const uint8_t* __restrict__ given, int64_t ld_given, uint8_t* __restrict__ codes, int64_t ld_codes,
    float* __restrict__ amax_out, int64_t ld_amax, uint8_t* __restrict__ clipped, uint8_t* __restrict__ flushed,
    int64_t ld_diag) {
  constexpr int ES = SRC_BF16 ? 2 : 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < nblocks; g += stride) {
    const int64_t row = g / nb, b = g - row * nb;
    const char* line = reinterpret_cast<const char*>(src) + row * ld_src * ES;
    Chunk<SRC_BF16> c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) load_chunk<SRC_BF16, VEC>(c[q], line, 32 * b + 8 * q, K);
    uint32_t v[32];
#pragma unroll
    for (int el = 0; el < 32; ++el) v[el] = value_bits<SRC_BF16>(c[el >> 3], el & 7);
    const int64_t rem = K - 32 * b;
    const int n_real = rem < 32 ? (int)rem : 32;
    const uint32_t sb = given[row * ld_given + b];
    uint32_t d[8], nclip, nflush;
    const uint32_t amax = F == kE4M3 ? encode_scaled_block<kE4M3>(v, sb, n_real, d, nclip, nflush)
                                     : encode_scaled_block<kE5M2>(v, sb, n_real, d, nclip, nflush);
    uint4* out = reinterpret_cast<uint4*>(codes + row * ld_codes + 32 * b);
    out[0] = make_uint4(d[0], d[1], d[2], d[3]);
    out[1] = make_uint4(d[4], d[5], d[6], d[7]);
    if (amax_out) amax_out[row * ld_amax + b] = __uint_as_float(amax);
    if (clipped) clipped[row * ld_diag + b] = (uint8_t)nclip;
    if (flushed) flushed[row * ld_diag + b] = (uint8_t)nflush;
  }
}

// Columnwise quantize with caller-owned scale bytes: the tile scheme of k_quant_cols.
template <int SRC_BF16, int F, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_cols_scaled(
    const void* __restrict__ src, int64_t rows, int64_t cols, int64_t ld_src, int64_t nb,
    const uint8_t* __restrict__ given, int64_t ld_given, uint8_t* __restrict__ codes, int64_t ld_codes,
    float* __restrict__ amax_out, int64_t ld_amax, uint8_t* __restrict__ clipped, uint8_t* __restrict__ flushed,
    int64_t ld_diag) {
  typedef typename std::conditional<SRC_BF16, uint16_t, uint32_t>::type E;
  constexpr int PW = kColTileCols * (int)sizeof(E) / 4 + 1;
  __shared__ uint32_t tile[kColTileRows * PW];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * kColTileCols;
  const E* s = reinterpret_cast<const E*>(src);
  for (int64_t ty = blockIdx.y; ty * kColTileRows < rows; ty += gridDim.y) {
    const int64_t r0 = ty * kColTileRows;
    constexpr int EPV = 16 / sizeof(E);
    constexpr int PPR = kColTileCols / EPV;
    for (int p = tid; p < kColTileRows * PPR; p += kThreads) {
      const int tr = p / PPR, tc = (p % PPR) * EPV;
      const int64_t r = r0 + tr, cc = c0 + tc;
      uint32_t* dst = &tile[tr * PW + tc * (int)sizeof(E) / 4];
      if (VEC && r < rows && cc + EPV <= cols) {
        const uint4 v = *reinterpret_cast<const uint4*>(s + r * ld_src + cc);
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
      } else {
        E e[EPV];
#pragma unroll
        for (int i = 0; i < EPV; ++i) e[i] = (r < rows && cc + i < cols) ? s[r * ld_src + cc + i] : (E)0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (SRC_BF16) dst[w] = (uint32_t)e[2 * w] | ((uint32_t)e[2 * w + 1] << 16);
          else dst[w] = (uint32_t)e[w];
        }
      }
    }
    __syncthreads();
    const int c = tid >> 2, kb = tid & 3;
    const int64_t col = c0 + c, b = r0 / 32 + kb;
    if (col < cols && b < nb) {
      uint32_t v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int row = 32 * kb + i;
        if (SRC_BF16) v[i] = (uint32_t)reinterpret_cast<const uint16_t*>(tile)[row * PW * 2 + c] << 16;
        else v[i] = tile[row * PW + c];
      }
      const int64_t rem = rows - 32 * b;
      const int n_real = rem < 32 ? (int)rem : 32;
      const uint32_t sb = given[col * ld_given + b];
      uint32_t out[8], nclip, nflush;
      const uint32_t amax = F == kE4M3 ? encode_scaled_block<kE4M3>(v, sb, n_real, out, nclip, nflush)
                                       : encode_scaled_block<kE5M2>(v, sb, n_real, out, nclip, nflush);
      uint4* dst = reinterpret_cast<uint4*>(codes + col * ld_codes + 32 * b);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      if (amax_out) amax_out[col * ld_amax + b] = __uint_as_float(amax);
      if (clipped) clipped[col * ld_diag + b] = (uint8_t)nclip;
      if (flushed) flushed[col * ld_diag + b] = (uint8_t)nflush;
    }
    __syncthreads();
  }
}
}  // namespace

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

template <int SRC_BF16, int F, int R>
static hipError_t quant_rows_t(const void* src, int64_t rows, int64_t K, int64_t ld_src, uint8_t* codes,
                               int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool flat, bool vec,
                               hipStream_t stream) {
  const int64_t nb = (K + 31) / 32;
  const int64_t nblocks = rows * nb;
  const int64_t wg_needed = (nblocks + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 256;   // beyond this, threads loop
  const int grid = (int)(wg_needed < cap ? wg_needed : cap);
  if (flat && vec)
    hipLaunchKernelGGL((k_quant_rows<SRC_BF16, F, true, true, R>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src, K,
                       nb, nblocks, codes, ld_codes, scales, ld_scales);
  else if (vec)
    hipLaunchKernelGGL((k_quant_rows<SRC_BF16, F, false, true, R>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src, K,
                       nb, nblocks, codes, ld_codes, scales, ld_scales);
  else
    hipLaunchKernelGGL((k_quant_rows<SRC_BF16, F, false, false, R>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src,
                       K, nb, nblocks, codes, ld_codes, scales, ld_scales);
  return hipGetLastError();
}

template <int R>
static hipError_t quant_rows_r(const void* src, int src_bf16, int64_t rows, int64_t K, int64_t ld_src, int fmt,
                               uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool flat,
                               bool vec, hipStream_t stream) {
  if (src_bf16) {
    if (fmt == kE4M3) return quant_rows_t<1, kE4M3, R>(src, rows, K, ld_src, codes, ld_codes, scales, ld_scales, flat, vec, stream);
    return quant_rows_t<1, kE5M2, R>(src, rows, K, ld_src, codes, ld_codes, scales, ld_scales, flat, vec, stream);
  }
  if (fmt == kE4M3) return quant_rows_t<0, kE4M3, R>(src, rows, K, ld_src, codes, ld_codes, scales, ld_scales, flat, vec, stream);
  return quant_rows_t<0, kE5M2, R>(src, rows, K, ld_src, codes, ld_codes, scales, ld_scales, flat, vec, stream);
}

hipError_t launch_quant_rows(const void* src, int src_bf16, int64_t rows, int64_t K, int64_t ld_src, int fmt,
                             int rule, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                             bool flat, bool vec, hipStream_t stream) {
  if (rule == kRuleOcp)
    return quant_rows_r<kRuleOcp>(src, src_bf16, rows, K, ld_src, fmt, codes, ld_codes, scales, ld_scales, flat, vec, stream);
  return quant_rows_r<kRuleCeil>(src, src_bf16, rows, K, ld_src, fmt, codes, ld_codes, scales, ld_scales, flat, vec, stream);
}

template <int SRC_BF16, int F, int R>
static hipError_t quant_cols_t(const void* src, int64_t rows, int64_t cols, int64_t ld_src, uint8_t* codes,
                               int64_t ld_codes, uint8_t* scales, int64_t ld_scales, hipStream_t stream) {
  constexpr int64_t ES = SRC_BF16 ? 2 : 4;
  const int64_t nb = (rows + 31) / 32;
  int64_t grid = 0;
  const ColTiles tiles = col_tiles(rows, cols, &grid);
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool buf = kColGroupRows * ld_src * ES < ((int64_t)1 << 31);
  const int vsc = (uintptr_t)scales % 16 == 0 && ld_scales % 16 == 0;
  if ((uintptr_t)src % 16 == 0 && (ld_src * ES) % 16 == 0 && (cols * ES) % 16 == 0 &&
      128 * ld_src * ES < ((int64_t)1 << 31)) {
    const int64_t gx = (cols + CtGeom<SRC_BF16>::TC - 1) / CtGeom<SRC_BF16>::TC;
    const int64_t ntiles = gx * ((rows + 127) / 128);
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    if (kXcds * per_xcd > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_quant_cols_lds<SRC_BF16, F, R, false>), dim3((unsigned)(kXcds * per_xcd)), dim3(kThreads),
                       0, stream, src, rows, cols, ld_src, nb, codes, ld_codes, scales, ld_scales, gx, ntiles, per_xcd,
                       (uint64_t)0);
    return hipGetLastError();
  }
  if (buf)
    hipLaunchKernelGGL((k_quant_cols<SRC_BF16, F, true, R>), dim3((unsigned)grid), dim3(kThreads), 0, stream, src,
                       rows, cols, ld_src, nb, codes, ld_codes, scales, ld_scales, tiles, vsc);
  else
    hipLaunchKernelGGL((k_quant_cols<SRC_BF16, F, false, R>), dim3((unsigned)grid), dim3(kThreads), 0, stream, src,
                       rows, cols, ld_src, nb, codes, ld_codes, scales, ld_scales, tiles, vsc);
  return hipGetLastError();
}

template <int R>
static hipError_t quant_cols_r(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, int fmt,
                               uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                               hipStream_t stream) {
  if (src_bf16) {
    if (fmt == kE4M3) return quant_cols_t<1, kE4M3, R>(src, rows, cols, ld_src, codes, ld_codes, scales, ld_scales, stream);
    return quant_cols_t<1, kE5M2, R>(src, rows, cols, ld_src, codes, ld_codes, scales, ld_scales, stream);
  }
  if (fmt == kE4M3) return quant_cols_t<0, kE4M3, R>(src, rows, cols, ld_src, codes, ld_codes, scales, ld_scales, stream);
  return quant_cols_t<0, kE5M2, R>(src, rows, cols, ld_src, codes, ld_codes, scales, ld_scales, stream);
}

hipError_t launch_quant_cols(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, int fmt,
                             int rule, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                             hipStream_t stream) {
  if (rule == kRuleOcp)
    return quant_cols_r<kRuleOcp>(src, src_bf16, rows, cols, ld_src, fmt, codes, ld_codes, scales, ld_scales, stream);
  return quant_cols_r<kRuleCeil>(src, src_bf16, rows, cols, ld_src, fmt, codes, ld_codes, scales, ld_scales, stream);
}

template <int SRC_BF16, int F>
static hipError_t quant_dual_t(const void* src, int64_t rows, int64_t cols, int64_t ld_src, uint8_t* rcodes,
                               int64_t ld_rc, uint8_t* rscales, int64_t ld_rs, uint8_t* ccodes, int64_t ld_cc,
                               uint8_t* cscales, int64_t ld_cs, bool vec, hipStream_t stream) {
  constexpr int64_t ES = SRC_BF16 ? 2 : 4;
  if ((uintptr_t)src % 16 == 0 && (ld_src * ES) % 16 == 0 && (cols * ES) % 16 == 0 &&
      128 * ld_src * ES < ((int64_t)1 << 31)) {
    const int64_t gx2 = (cols + 127) / 128;
    const int64_t ntiles = gx2 * ((rows + 127) / 128);
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    if (kXcds * per_xcd > 0x7FFFFFFF) return hipErrorInvalidValue;
    constexpr int lds = 128 * 128 * (int)ES;
    auto kern = k_quant_dual_lds<SRC_BF16, F>;
    if (lds > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
            hipSuccess)
      return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)(kXcds * per_xcd)), dim3(kThreads), lds, stream, src, rows, cols, ld_src,
                       rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs, gx2, ntiles, per_xcd);
    return hipGetLastError();
  }
  const int64_t gx = (cols + kColTileCols - 1) / kColTileCols;
  int64_t gy = (rows + kColTileRows - 1) / kColTileRows;
  if (gy > 65535) gy = 65535;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL((k_quant_dual<SRC_BF16, F, true>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, stream,
                       src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs);
  else
    hipLaunchKernelGGL((k_quant_dual<SRC_BF16, F, false>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, stream,
                       src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs);
  return hipGetLastError();
}

hipError_t launch_quant_dual(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, int fmt,
                             uint8_t* rcodes, int64_t ld_rc, uint8_t* rscales, int64_t ld_rs, uint8_t* ccodes,
                             int64_t ld_cc, uint8_t* cscales, int64_t ld_cs, bool vec, hipStream_t stream) {
  if (src_bf16) {
    if (fmt == kE4M3)
      return quant_dual_t<1, kE4M3>(src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs, vec, stream);
    return quant_dual_t<1, kE5M2>(src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs, vec, stream);
  }
  if (fmt == kE4M3)
    return quant_dual_t<0, kE4M3>(src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs, vec, stream);
  return quant_dual_t<0, kE5M2>(src, rows, cols, ld_src, rcodes, ld_rc, rscales, ld_rs, ccodes, ld_cc, cscales, ld_cs, vec, stream);
}

template <int SRC_BF16, int F>
static hipError_t quant_sr_t(const void* src, int64_t rows, int64_t cols, int64_t ld_src, bool colwise,
                             uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool vec,
                             uint64_t seed, hipStream_t stream) {
  if (!colwise) {
    const int64_t nb = (cols + 31) / 32, nblocks = rows * nb;
    const int64_t wg_needed = (nblocks + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)device_cu_count() * 256;
    const int grid = (int)(wg_needed < cap ? wg_needed : cap);
    if (vec)
      hipLaunchKernelGGL((k_quant_rows_sr<SRC_BF16, F, true>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src, cols,
                         nb, nblocks, codes, ld_codes, scales, ld_scales, seed);
    else
      hipLaunchKernelGGL((k_quant_rows_sr<SRC_BF16, F, false>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src,
                         cols, nb, nblocks, codes, ld_codes, scales, ld_scales, seed);
    return hipGetLastError();
  }
  const int64_t nb = (rows + 31) / 32;
  constexpr int64_t ES = SRC_BF16 ? 2 : 4;
  if ((uintptr_t)src % 16 == 0 && (ld_src * ES) % 16 == 0 && (cols * ES) % 16 == 0 &&
      128 * ld_src * ES < ((int64_t)1 << 31)) {
    // the columnwise LDS tile kernel of quant_cols_t with the stochastic encoder
    const int64_t tgx = (cols + CtGeom<SRC_BF16>::TC - 1) / CtGeom<SRC_BF16>::TC;
    const int64_t ntiles = tgx * ((rows + 127) / 128);
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    if (kXcds * per_xcd > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_quant_cols_lds<SRC_BF16, F, kRuleCeil, true>), dim3((unsigned)(kXcds * per_xcd)),
                       dim3(kThreads), 0, stream, src, rows, cols, ld_src, nb, codes, ld_codes, scales, ld_scales,
                       tgx, ntiles, per_xcd, seed);
    return hipGetLastError();
  }
  const int64_t gx = (cols + kColTileCols - 1) / kColTileCols;
  int64_t gy = (rows + kColTileRows - 1) / kColTileRows;
  if (gy > 65535) gy = 65535;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL((k_quant_cols_sr<SRC_BF16, F, true>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       stream, src, rows, cols, ld_src, nb, codes, ld_codes, scales, ld_scales, seed);
  else
    hipLaunchKernelGGL((k_quant_cols_sr<SRC_BF16, F, false>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       stream, src, rows, cols, ld_src, nb, codes, ld_codes, scales, ld_scales, seed);
  return hipGetLastError();
}

template <int SRC_BF16, int F>
static hipError_t quant_scaled_t(const void* src, int64_t rows, int64_t cols, int64_t ld_src, bool colwise,
                                 const uint8_t* given, int64_t ld_given, uint8_t* codes, int64_t ld_codes,
                                 float* amax, int64_t ld_amax, uint8_t* clipped, uint8_t* flushed, int64_t ld_diag,
                                 bool vec, hipStream_t stream) {
  if (!colwise) {
    const int64_t nb = (cols + 31) / 32, nblocks = rows * nb;
    const int64_t wg_needed = (nblocks + kThreads - 1) / kThreads;
    const int64_t cap = (int64_t)device_cu_count() * 256;
    const int grid = (int)(wg_needed < cap ? wg_needed : cap);
    if (vec)
      hipLaunchKernelGGL((k_quant_rows_scaled<SRC_BF16, F, true>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src,
                         cols, nb, nblocks, given, ld_given, codes, ld_codes, amax, ld_amax, clipped, flushed, ld_diag);
    else
      hipLaunchKernelGGL((k_quant_rows_scaled<SRC_BF16, F, false>), dim3(grid), dim3(kThreads), 0, stream, src, ld_src,
                         cols, nb, nblocks, given, ld_given, codes, ld_codes, amax, ld_amax, clipped, flushed, ld_diag);
    return hipGetLastError();
  }
  const int64_t nb = (rows + 31) / 32;
  const int64_t gx = (cols + kColTileCols - 1) / kColTileCols;
  int64_t gy = (rows + kColTileRows - 1) / kColTileRows;
  if (gy > 65535) gy = 65535;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL((k_quant_cols_scaled<SRC_BF16, F, true>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       stream, src, rows, cols, ld_src, nb, given, ld_given, codes, ld_codes, amax, ld_amax, clipped,
                       flushed, ld_diag);
  else
    hipLaunchKernelGGL((k_quant_cols_scaled<SRC_BF16, F, false>), dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                       stream, src, rows, cols, ld_src, nb, given, ld_given, codes, ld_codes, amax, ld_amax, clipped,
                       flushed, ld_diag);
  return hipGetLastError();
}

hipError_t launch_quant_scaled(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, bool colwise,
                               int fmt, const uint8_t* given, int64_t ld_given, uint8_t* codes, int64_t ld_codes,
                               float* amax, int64_t ld_amax, uint8_t* clipped, uint8_t* flushed, int64_t ld_diag,
                               bool vec, hipStream_t stream) {
  if (src_bf16) {
    if (fmt == kE4M3)
      return quant_scaled_t<1, kE4M3>(src, rows, cols, ld_src, colwise, given, ld_given, codes, ld_codes, amax, ld_amax,
                                      clipped, flushed, ld_diag, vec, stream);
    return quant_scaled_t<1, kE5M2>(src, rows, cols, ld_src, colwise, given, ld_given, codes, ld_codes, amax, ld_amax,
                                    clipped, flushed, ld_diag, vec, stream);
  }
  if (fmt == kE4M3)
    return quant_scaled_t<0, kE4M3>(src, rows, cols, ld_src, colwise, given, ld_given, codes, ld_codes, amax, ld_amax,
                                    clipped, flushed, ld_diag, vec, stream);
  return quant_scaled_t<0, kE5M2>(src, rows, cols, ld_src, colwise, given, ld_given, codes, ld_codes, amax, ld_amax,
                                  clipped, flushed, ld_diag, vec, stream);
}

hipError_t launch_quant_sr(const void* src, int src_bf16, int64_t rows, int64_t cols, int64_t ld_src, bool colwise,
                           int fmt, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, bool vec,
                           uint64_t seed, hipStream_t stream) {
  if (src_bf16) {
    if (fmt == kE4M3)
      return quant_sr_t<1, kE4M3>(src, rows, cols, ld_src, colwise, codes, ld_codes, scales, ld_scales, vec, seed, stream);
    return quant_sr_t<1, kE5M2>(src, rows, cols, ld_src, colwise, codes, ld_codes, scales, ld_scales, vec, seed, stream);
  }
  if (fmt == kE4M3)
    return quant_sr_t<0, kE4M3>(src, rows, cols, ld_src, colwise, codes, ld_codes, scales, ld_scales, vec, seed, stream);
  return quant_sr_t<0, kE5M2>(src, rows, cols, ld_src, colwise, codes, ld_codes, scales, ld_scales, vec, seed, stream);
}

}  // namespace mxq
