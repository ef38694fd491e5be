// Stable least-significant-digit radix pass over (key, value) pairs, the
// device form of the counting sort the Day 40 page ("One iteration, three
// shapes of work") runs on the host: per 8-bit digit, a histogram of the
// digit per tile, an exclusive scan over the digit-major histogram matrix,
// and a scatter in which every element keeps its order among equal digits.
//
// Tile = 256 lanes x 16 items = 4096 elements.  Each wavefront owns 1024
// consecutive elements and walks them as 16 rounds of 64 consecutive
// elements, so the (round, lane) order is the element order.  The rank of an
// element among equal digits in its round comes from eight ballots (one per
// digit bit); a per-wavefront LDS counter per digit carries the count across
// rounds.  Elements are then reordered in LDS by (digit, order) and written
// out in digit runs, so global writes are contiguous within each run.
#pragma once

#include "common.hpp"

namespace pr {

constexpr int kRadixBits = 8;
constexpr int kRadixDigits = 1 << kRadixBits;
constexpr int kRadixItems = 16;
constexpr int kRadixTile = kBlock * kRadixItems;

// Where the pass reads its pairs from.
enum RadixMode : int {
    // First transpose pass: key = target id out_col_idx[e]; value = the source
    // row u that owns edge e (from the row starts inside e's tile, within the
    // tile's row range from k_tile_rows; see stage_owner_rows).
    kFromOutCsr = 0,
    // Later passes: keys_in[e], vals_in[e].
    kFromPairs = 1,
    // Vertex keys: key = keys[i], value = i.
    kFromKeys = 2,
    // Keys only, first pass: key = target id out_col_idx[i] (range-checked).
    kFromTargets = 3,
    // Edges by tile: key = target plan id keys[i], value = vals[i], digit taken
    // from tile_of(key) (targets are plan ids, valid by construction); every
    // pass reads pairs this way, so the sorted keys are still targets.
    kFromTileTargets = 4,
    // Edges by tile, first pass over a CSR in plan order: key = target plan
    // id keys[i] (the column array), digit from tile_of(key); value = the row
    // that owns edge i, found from row_ptr as in kFromOutCsr.
    kFromTileCsr = 5,
};

// Tiles of the plan: consecutive plan-id segments (one per degree bucket,
// hub bucket first), each cut into blocks of 2^shift rows.
constexpr int kTileSegments = 5;
struct TileMap {
    int32_t start[kTileSegments + 1];  // first plan id of each segment; [kTileSegments] = n
    int32_t tile0[kTileSegments];      // first tile of each segment
    int32_t shift[kTileSegments];      // log2 of the segment's rows per tile
};

// Tile of plan id v and v's row offset in it.  The segment is the last one
// whose start is <= v (an empty segment shares its start with the next,
// which then wins); its fields are picked with selects rather than an index,
// so they stay in scalar registers instead of being reloaded per lane.
struct TileSpot {
    int32_t tile;
    int32_t offset;
};

__host__ __device__ inline TileSpot tile_locate(const TileMap& m, int32_t v) {
    int32_t start = m.start[0], tile0 = m.tile0[0], shift = m.shift[0];
#pragma unroll
    for (int j = 1; j < kTileSegments; ++j) {
        const bool in = v >= m.start[j];
        start = in ? m.start[j] : start;
        tile0 = in ? m.tile0[j] : tile0;
        shift = in ? m.shift[j] : shift;
    }
    const int32_t rel = v - start;
    return TileSpot{tile0 + (rel >> shift), rel & ((1 << shift) - 1)};
}

__host__ __device__ inline int32_t tile_of(const TileMap& m, int32_t v) { return tile_locate(m, v).tile; }

struct RadixIn {
    int64_t count;                 // elements
    int32_t n;                     // vertices
    const int32_t* keys;           // kFromOutCsr: out_col_idx; other modes: keys
    const int32_t* vals;           // kFromPairs, kFromTileTargets
    const int32_t* row_ptr;        // kFromOutCsr, kFromTileCsr: the row pointers
    const int32_t* tile_row;       // kFromOutCsr, kFromTileCsr: [T + 1] from k_tile_rows
    TileMap tiles;                 // kFromTileTargets, kFromTileCsr
    int32_t tile_base = 0;         // kFromTileTargets, kFromTileCsr: the digit is
    int32_t tile_cap = INT32_MAX;  //   min(tile_of(key) - tile_base, tile_cap)
    uint32_t* error;               // set to 1 when an input index is out of range
};

// Largest r in [lo, hi] with row_ptr[r] <= e (the row owning edge e when
// row_ptr is a valid CSR).  Clamped, so malformed input cannot index out of
// bounds.
__device__ __forceinline__ int32_t owner_row(const int32_t* __restrict__ rp, int64_t e, int32_t lo,
                                             int32_t hi) {
    while (lo < hi) {
        int32_t mid = lo + (hi - lo + 1) / 2;
        if ((int64_t)rp[mid] <= e)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// The key of element i as stored (no checks).
__device__ __forceinline__ int32_t radix_load(const RadixIn& in, int64_t i) { return in.keys[i]; }

// The key a pass uses for a loaded value k: targets read from a caller's CSR
// are range-checked (an out-of-range one is clamped, so it cannot index out
// of bounds later, and sets `bad`).  The caller raises the error flag once,
// with report_bad: a store in the per-item loop would make the compiler
// reload the kernel's arguments after every item.
template <int MODE>
__device__ __forceinline__ int32_t radix_check(const RadixIn& in, int32_t k, bool& bad) {
    if (MODE == kFromOutCsr || MODE == kFromTargets) {
        const bool out = (uint32_t)k >= (uint32_t)in.n;
        bad |= out;
        k = out ? (k < 0 ? 0 : in.n - 1) : k;
    }
    return k;
}

template <int MODE>
__device__ __forceinline__ void report_bad(const RadixIn& in, bool bad) {
    if ((MODE == kFromOutCsr || MODE == kFromTargets) && bad) *in.error = 1u;
}

// The digit a pass sorts by: of the key, or of the key's tile.
template <int MODE>
__device__ __forceinline__ uint32_t radix_digit(const RadixIn& in, int32_t k, int shift) {
    uint32_t d = (uint32_t)k;
    if (MODE == kFromTileTargets || MODE == kFromTileCsr) {
        const int32_t t = tile_of(in.tiles, k) - in.tile_base;
        d = (uint32_t)(t < in.tile_cap ? t : in.tile_cap);
    }
    return (d >> shift) & (kRadixDigits - 1);
}

// The digit of a tile-keyed pass, with the tile map staged in LDS: seg[j] =
// {start, first tile - tile_base, shift} of segment j.  The segment is the
// number of segment starts after the first that are <= k (an empty segment
// shares its start with the next, which then counts too), so one LDS read
// replaces the chain of selects in tile_of, each of which costs two vector
// instructions when its operands are kernel arguments (an instruction may
// read one scalar register besides the condition).
struct SegRow {
    int32_t start, tile0, shift, pad;
};
// seg[j] = {start[j], tile0[j] - tile_base, shift[j]}, from the first
// kTileSegments lanes; read after a barrier
__device__ __forceinline__ void stage_segments(SegRow* seg, const TileMap& m, int32_t tile_base) {
    if (threadIdx.x < kTileSegments)
        seg[threadIdx.x] = SegRow{m.start[threadIdx.x], m.tile0[threadIdx.x] - tile_base,
                                  m.shift[threadIdx.x], 0};
}
__device__ __forceinline__ int32_t seg_tile(const SegRow* seg, const TileMap& m, int32_t k) {
    int32_t j = 0;
#pragma unroll
    for (int i = 1; i < kTileSegments; ++i) j += k >= m.start[i] ? 1 : 0;
    const SegRow r = seg[j];
    return r.tile0 + ((k - r.start) >> r.shift);
}
__device__ __forceinline__ uint32_t tile_digit(const SegRow* seg, const RadixIn& in, int32_t k,
                                               int shift) {
    const int32_t t = seg_tile(seg, in.tiles, k);
    return ((uint32_t)(t < in.tile_cap ? t : in.tile_cap) >> shift) & (kRadixDigits - 1);
}

// Lanes of the wavefront whose digit equals this lane's (among `valid` lanes),
// from one ballot per digit bit: with m the bit as a lane mask (0 or all
// ones), peers &= ~(ballot(m) ^ m), one three-input bitwise instruction per
// 32-bit half (truth table 0x90 over (peers, votes, m): peers and votes equal
// to m).  Four vector instructions per bit; the two-way select it replaces
// took nine.
__device__ __forceinline__ uint64_t digit_peers(uint32_t dg, bool valid) {
    const uint64_t all = __ballot(valid);
    uint32_t lo = (uint32_t)all, hi = (uint32_t)(all >> 32);
#pragma unroll
    for (int b = 0; b < kRadixBits; ++b) {
        const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int32_t)dg, b, 1);
        const uint64_t votes = __builtin_amdgcn_uicmp(m, 0u, 33);  // 33: not equal
        lo = __builtin_amdgcn_bitop3_b32(lo, (uint32_t)votes, m, 0x90);
        hi = __builtin_amdgcn_bitop3_b32(hi, (uint32_t)(votes >> 32), m, 0x90);
    }
    return ((uint64_t)hi << 32) | lo;
}

// Workgroups are dealt to the eight XCDs in turn (workgroup b to XCD b mod 8)
// and every XCD has an L2 of its own.  Tiles t and t + 1 write neighbouring
// words of every histogram row and neighbouring pieces of each digit's
// output run, often parts of one cache line, so the histogram and scatter
// passes give each XCD a contiguous range of tiles, taken in order: the
// pieces of a line then meet in one L2 instead of leaving partial lines in
// several.  (On RMAT-23: the later scatter passes 1.41 -> 1.04 ms, the
// histograms 0.30 -> 0.25 ms.  k_permute_rows keeps the dealt order: given
// contiguous ranges it ran slower.)
// A bijection of [0, T): XCD x gets floor(T / 8) tiles, plus one if x < T mod 8.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t T) {
    const int64_t x = b % kXcds, j = b / kXcds, q = T / kXcds, r = T % kXcds;
    return x * q + (x < r ? x : r) + j;
}

// Counts digits into the LDS histogram h, one item at a time.  Graph keys
// are skewed: many lanes of a round often hold digit 0 (the low ids of a
// power-law graph, or the hub tiles), and LDS adds to one address
// serialize, so digits below kRegDigits are counted in registers and added
// once per wavefront by flush(), which every lane calls.
struct DigitCounter {
    static constexpr int kRegDigits = 4;
    uint32_t reg[kRegDigits] = {};
    __device__ __forceinline__ void add(uint32_t dg, uint32_t* h, uint32_t c = 1u) {
        if (dg < (uint32_t)kRegDigits) {
#pragma unroll
            for (int j = 0; j < kRegDigits; ++j) reg[j] += dg == (uint32_t)j ? c : 0u;
        } else {
            atomicAdd(&h[dg], c);
        }
    }
    __device__ __forceinline__ void flush(uint32_t* h) {
#pragma unroll
        for (int j = 0; j < kRegDigits; ++j) {
            const uint32_t c = wave_sum(reg[j]);
            if (lane_id() == 0 && c) atomicAdd(&h[j], c);
        }
    }
};

// Histogram of one digit per tile, stored digit-major: hist[digit * T + tile].
// A lane takes kRadixItems consecutive keys (four 16-byte loads) and adds
// each run of equal digits once: a CSR's rows hold their targets in
// increasing order, so neighbouring keys often share their high digits, and
// lanes adding one at a time to the same LDS counter serialize.
template <int MODE>
__global__ __launch_bounds__(kBlock) void k_radix_hist(RadixIn in, int shift, int64_t T,
                                                       uint32_t* __restrict__ hist) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    __shared__ uint32_t h[kRadixDigits];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t tile = xcd_tile(blockIdx.x, T);
    const int64_t i0 = tile * kRadixTile + threadIdx.x * kRadixItems;
    const int64_t left = in.count - i0;  // keys of this lane: min(left, kRadixItems)
    int32_t k[kRadixItems];
    // (16-byte loads when the keys are 16-byte aligned: scratch always is, a
    // caller's CSR or a sub-range of scratch need not be)
    if (left >= kRadixItems && (reinterpret_cast<uintptr_t>(in.keys) & 15u) == 0) {
#pragma unroll
        for (int q = 0; q < kRadixItems / 4; ++q) {
            const i32x4 v = *(const i32x4*)(in.keys + i0 + 4 * q);
            k[4 * q] = v.x;
            k[4 * q + 1] = v.y;
            k[4 * q + 2] = v.z;
            k[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int r = 0; r < kRadixItems; ++r) k[r] = r < left ? radix_load(in, i0 + r) : 0;
    }
    DigitCounter dc;
    uint32_t cur = 0, run = 0;
    bool bad = false;
#pragma unroll
    for (int r = 0; r < kRadixItems; ++r) {
        if (r >= left) break;
        const uint32_t dg = radix_digit<MODE>(in, radix_check<MODE>(in, k[r], bad), shift);
        if (run > 0 && dg != cur) {
            dc.add(cur, h, run);
            run = 0;
        }
        cur = dg;
        ++run;
    }
    if (run > 0) dc.add(cur, h, run);
    report_bad<MODE>(in, bad);
    dc.flush(h);
    __syncthreads();
    hist[(int64_t)threadIdx.x * T + tile] = h[threadIdx.x];
}

// Owner rows of a first-pass tile, when the rows it touches are at most
// kRadixTile: own[i] = the row of edge base + i, for i < count.  Each row
// that starts inside the tile marks its first slot (of rows that start at
// the same slot, the last one wins: the others are empty), and an inclusive
// max-scan carries the marks forward; slot 0 belongs to `lo`, the owner of
// the tile's first edge.  The scan: every lane takes the maximum of its
// kRadixItems consecutive slots, a workgroup-wide exclusive max-scan of
// those gives each lane its carry, and the lane sweeps its slots again from
// it.  (Sixteen 64-slot rounds per wavefront, each waiting for the last
// one's carry, cost about four times as much.)  `wave_max` is kWaves words
// of LDS.  Slot i lives at own[owner_slot(i)], a bijection of [0, 4096) that
// keeps the lane-strided sweeps (lane t: slots 16t..16t+15) and the
// consecutive reads of the ranking loop in 64 distinct LDS banks: unswizzled,
// a strided sweep put a wavefront's reads in four.  Contains barriers: call
// from every lane.
__device__ __forceinline__ int owner_slot(int i) { return i ^ ((i >> 4) & 63); }

// The scan half of stage_owner_rows: own[owner_slot(i)], i < count, holds a
// mark (a row) or -1; afterwards every slot holds the largest mark at or
// before it.  Contains barriers: call from every lane.
__device__ __forceinline__ void owner_max_scan(int count, int32_t* own, int32_t* wave_max) {
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int i0 = tid * kRadixItems;
    int32_t m = -1;
#pragma unroll
    for (int j = 0; j < kRadixItems; ++j)
        if (i0 + j < count) m = max(m, own[owner_slot(i0 + j)]);
    // exclusive max-scan of the lanes' maxima, in lane order
    int32_t incl = m;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int32_t t = __shfl_up(incl, off, kWave);
        if (lane >= off) incl = max(incl, t);
    }
    int32_t carry = __shfl_up(incl, 1, kWave);
    if (lane == 0) carry = -1;
    if (lane == kWave - 1) wave_max[wave] = incl;
    __syncthreads();
    for (int w = 0; w < wave; ++w) carry = max(carry, wave_max[w]);
#pragma unroll
    for (int j = 0; j < kRadixItems; ++j) {
        if (i0 + j < count) {
            carry = max(carry, own[owner_slot(i0 + j)]);
            own[owner_slot(i0 + j)] = carry;
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void stage_owner_rows(const int32_t* __restrict__ rp, int64_t base,
                                                 int count, int32_t lo, int32_t hi, int32_t* own,
                                                 int32_t* wave_max) {
    const int tid = threadIdx.x;
    for (int i = tid; i < count; i += kBlock) own[owner_slot(i)] = i == 0 ? lo : -1;
    __syncthreads();
    for (int32_t r = lo + 1 + tid; r <= hi; r += kBlock) {
        const int64_t p = (int64_t)rp[r] - base;
        if (p > 0 && p < count) atomicMax(&own[owner_slot((int)p)], r);  // in range for a valid row_ptr
    }
    __syncthreads();
    owner_max_scan(count, own, wave_max);
}

// Stable scatter.  `scanned` is the exclusive scan of the digit-major
// histogram.  Keys are written only when keys_out is not null (with KEY16,
// as uint16 words holding each key's low 16 bits); values are carried only
// when VALS.
template <int MODE, bool VALS = true, bool KEY16 = false>
__global__ __launch_bounds__(kBlock) void k_radix_scatter(RadixIn in, int shift, int64_t T,
                                                          const uint32_t* __restrict__ scanned,
                                                          int32_t* __restrict__ keys_out,
                                                          int32_t* __restrict__ vals_out) {
    __shared__ uint32_t wave_count[kWaves][kRadixDigits];
    __shared__ uint32_t digit_start[kRadixDigits];
    __shared__ uint32_t global_start[kRadixDigits];
    __shared__ int32_t s_key[kRadixTile];
    __shared__ int32_t s_val[kRadixTile];
    __shared__ uint32_t scan_tmp[kWaves + 1];
    __shared__ SegRow seg[kTileSegments];
    constexpr bool kTileKeys = MODE == kFromTileTargets || MODE == kFromTileCsr;
    // the digit of key k (after the first barrier below)
    auto digit = [&](int32_t k) -> uint32_t {
        if constexpr (kTileKeys)
            return tile_digit(seg, in, k, shift);
        else
            return radix_digit<MODE>(in, k, shift);
    };

    // A tile-keyed pass with keys below 2^24 (plan ids of a graph with at
    // most that many vertices) keeps each key's digit in its top byte in LDS,
    // so the write-out does not look the tile up again.
    constexpr int kPackShift = 32 - kRadixBits;
    const bool packed = kTileKeys && in.n <= (1 << kPackShift);

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    if (kTileKeys) stage_segments(seg, in.tiles, in.tile_base);
    const int64_t tile = xcd_tile(blockIdx.x, T);
    const int64_t base = tile * kRadixTile;
    const int count = (int)((in.count - base) < kRadixTile ? (in.count - base) : kRadixTile);

#pragma unroll
    for (int w = 0; w < kWaves; ++w) wave_count[w][tid] = 0;

    int32_t key[kRadixItems], val[kRadixItems];
    uint32_t rank[kRadixItems];
    // all of the lane's loads first (an index past the end reloads the last
    // element, which is then ignored), so they overlap
    constexpr bool kLoadVals = VALS && (MODE == kFromPairs || MODE == kFromTileTargets);
#pragma unroll
    for (int r = 0; r < kRadixItems; ++r) {
        const int idx = wave * (kWave * kRadixItems) + r * kWave + lane;
        const int64_t g = base + (idx < count ? idx : count - 1);
        key[r] = radix_load(in, g);
        if (kLoadVals) val[r] = in.vals[g];
    }
    // First pass: the rows that own the tile's edges lie in [row_lo, row_hi]
    // (clamped, so a malformed row_ptr cannot index out of bounds).  Their
    // owner rows come from LDS when there are few enough of them (a tile
    // inside a long run of empty rows searches row_ptr per edge instead).
    // s_val is free until the reorder below.  The loads above stay in flight
    // meanwhile: the barriers here wait for LDS only.
    constexpr bool kRows = MODE == kFromOutCsr || MODE == kFromTileCsr;  // values: owner rows
    int32_t row_lo = 0, row_hi = 0;
    if (kRows) {
        row_lo = min(max(in.tile_row[tile], 0), in.n - 1);
        row_hi = min(max(in.tile_row[tile + 1], row_lo), in.n - 1);
    }
    const bool staged_rows = kRows && VALS && row_hi - row_lo < kRadixTile;
    if (staged_rows)
        stage_owner_rows(in.row_ptr, base, count, row_lo, row_hi, s_val, (int32_t*)scan_tmp);
    else
        __syncthreads();  // the wave counters' clearing

    bool bad = false;
#pragma unroll
    for (int r = 0; r < kRadixItems; ++r) {
        const int idx = wave * (kWave * kRadixItems) + r * kWave + lane;
        const bool valid = idx < count;
        int32_t k = 0, v = 0;
        if (valid) {
            const int64_t g = base + idx;
            k = radix_check<MODE>(in, key[r], bad);
            if (!VALS)
                v = 0;
            else if (kRows)
                v = staged_rows ? s_val[owner_slot(idx)] : owner_row(in.row_ptr, g, row_lo, row_hi);
            else if (kLoadVals)
                v = val[r];
            else
                v = (int32_t)g;  // kFromKeys: the index itself
        }
        const uint32_t dg = digit(k);
        const uint64_t peers = digit_peers(dg, valid);
        const uint32_t below = lanes_below(peers);
        uint32_t prior = 0;
        if (valid) prior = wave_count[wave][dg];
        if (valid && below == 0) wave_count[wave][dg] = prior + (uint32_t)__popcll(peers);
        key[r] = k;
        val[r] = v;
        rank[r] = prior + below;
    }
    report_bad<MODE>(in, bad);
    __syncthreads();

    {  // lane tid owns digit tid: per-wavefront prefixes and the tile's digit starts
        uint32_t c[kWaves], tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            c[w] = wave_count[w][tid];
            wave_count[w][tid] = tot;
            tot += c[w];
        }
        uint32_t all;
        digit_start[tid] = block_exclusive_scan(tot, &all, scan_tmp);
        global_start[tid] = scanned[(int64_t)tid * T + tile];
    }
    __syncthreads();

#pragma unroll
    for (int r = 0; r < kRadixItems; ++r) {
        const int idx = wave * (kWave * kRadixItems) + r * kWave + lane;
        if (idx < count) {
            const uint32_t dg = digit(key[r]);
            const uint32_t pos = digit_start[dg] + wave_count[wave][dg] + rank[r];
            s_key[pos] = packed ? (int32_t)((uint32_t)key[r] | (dg << kPackShift)) : key[r];
            if (VALS) s_val[pos] = val[r];
        }
    }
    __syncthreads();

    for (int i = tid; i < count; i += kBlock) {
        int32_t k = s_key[i];
        uint32_t dg;
        if (packed) {
            dg = (uint32_t)k >> kPackShift;
            k &= (1 << kPackShift) - 1;
        } else {
            dg = digit(k);
        }
        const int64_t o = (int64_t)global_start[dg] + (i - (int64_t)digit_start[dg]);
        if (KEY16)
            reinterpret_cast<uint16_t*>(keys_out)[o] = (uint16_t)k;
        else if (keys_out)
            keys_out[o] = k;
        if (VALS) vals_out[o] = s_val[i];
    }
}

// Number of tiles for `count` elements.
inline int64_t radix_tiles(int64_t count) { return ceil_div(count > 0 ? count : 1, kRadixTile); }

static_assert(kBlock == kRadixDigits, "one lane per digit in the scatter's digit phase");

// Scratch for a full LSD sort of `count` pairs.
struct RadixWs {
    uint32_t* hist;      // [256 * T]
    uint32_t* scanned;   // [256 * T + 1]
    int32_t* key[2];     // [count] each, ping-pong
    int32_t* val[2];
    void* scan_ws;
};

inline RadixWs radix_carve(Carver& c, int64_t count) {
    RadixWs w{};
    const int64_t T = radix_tiles(count);
    w.hist = c.take<uint32_t>((size_t)(kRadixDigits * T));
    w.scanned = c.take<uint32_t>((size_t)(kRadixDigits * T + 1));
    for (int i = 0; i < 2; ++i) {
        w.key[i] = c.take<int32_t>((size_t)count);
        w.val[i] = c.take<int32_t>((size_t)count);
    }
    // big enough for the histogram scan and for a scan over `count` items
    const int64_t scan_n = kRadixDigits * T > count ? kRadixDigits * T : count;
    w.scan_ws = c.base ? c.base + c.used : nullptr;
    c.used += align_up(scan_workspace_bytes(scan_n));
    return w;
}

// Stable LSD sort of `count` >= 1 pairs by the low `bits` bits of the key (at
// least one pass).  Pass 0 reads its pairs per MODE; later passes read the
// previous pass's output.  The sorted values end in vals_out; the sorted keys
// are left in *keys_sorted (one of the scratch buffers).
template <int MODE>
int radix_sort(RadixIn in, int bits, int32_t* vals_out, const RadixWs& w, int32_t** keys_sorted,
               hipStream_t stream) {
    constexpr int kLater = MODE == kFromTileTargets ? kFromTileTargets : kFromPairs;
    if (in.count < 1) return fail(PR_ERR_ARG, "radix sort of %lld elements", (long long)in.count);
    const int64_t T = radix_tiles(in.count);
    int passes = (bits + kRadixBits - 1) / kRadixBits;
    if (passes < 1) passes = 1;
    for (int p = 0; p < passes; ++p) {
        const int shift = p * kRadixBits;
        const bool last = p == passes - 1;
        int32_t* kout = w.key[p & 1];
        int32_t* vout = last ? vals_out : w.val[p & 1];
        if (p == 0)
            k_radix_hist<MODE><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, shift, T, w.hist);
        else
            k_radix_hist<kLater><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, shift, T, w.hist);
        PR_LAUNCHED("radix histogram");
        PR_TRY(scan_exclusive(w.hist, w.scanned, kRadixDigits * T, w.scan_ws, stream));
        if (p == 0)
            k_radix_scatter<MODE><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, shift, T, w.scanned,
                                                                             kout, vout);
        else
            k_radix_scatter<kLater><<<dim3((unsigned)T), kBlock, 0, stream>>>(
                in, shift, T, w.scanned, kout, vout);
        PR_LAUNCHED("radix scatter");
        in.keys = kout;
        in.vals = vout;
        *keys_sorted = kout;
    }
    return PR_OK;
}

// Stable LSD sort of `count` >= 1 pairs (read per MODE) by the low `bits`
// bits of the digit, in max(2, ceil(bits / 8)) passes: pass p writes the
// scratch pair p & 1, the last pass (keys_out, vals_out).  The input may be
// the output range itself (the first pass writes scratch); the scratch pairs
// must not overlap the input, the output or each other.
template <int MODE>
int radix_sort_to(RadixIn in, int bits, int32_t* keys_out, int32_t* vals_out,
                  int32_t* const scratch_keys[2], int32_t* const scratch_vals[2], const RadixWs& w,
                  hipStream_t stream) {
    if (in.count < 1) return fail(PR_ERR_ARG, "radix sort of %lld elements", (long long)in.count);
    const int64_t T = radix_tiles(in.count);
    int passes = (bits + kRadixBits - 1) / kRadixBits;
    if (passes < 2) passes = 2;
    for (int p = 0; p < passes; ++p) {
        const bool last = p == passes - 1;
        int32_t* kout = last ? keys_out : scratch_keys[p & 1];
        int32_t* vout = last ? vals_out : scratch_vals[p & 1];
        k_radix_hist<MODE><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, p * kRadixBits, T, w.hist);
        PR_LAUNCHED("radix histogram");
        PR_TRY(scan_exclusive(w.hist, w.scanned, kRadixDigits * T, w.scan_ws, stream));
        k_radix_scatter<MODE><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, p * kRadixBits, T, w.scanned,
                                                                         kout, vout);
        PR_LAUNCHED("radix scatter");
        in.keys = kout;
        in.vals = vout;
    }
    return PR_OK;
}

// Stable LSD sort of `count` >= 1 keys alone by their low `bits` bits; pass 0
// reads keys per MODE.  The sorted keys are left in *keys_sorted.
template <int MODE>
int radix_sort_keys(RadixIn in, int bits, const RadixWs& w, int32_t** keys_sorted,
                    hipStream_t stream) {
    if (in.count < 1) return fail(PR_ERR_ARG, "radix sort of %lld elements", (long long)in.count);
    const int64_t T = radix_tiles(in.count);
    int passes = (bits + kRadixBits - 1) / kRadixBits;
    if (passes < 1) passes = 1;
    for (int p = 0; p < passes; ++p) {
        const int shift = p * kRadixBits;
        int32_t* kout = w.key[p & 1];
        if (p == 0)
            k_radix_hist<MODE><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, shift, T, w.hist);
        else
            k_radix_hist<kFromPairs><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, shift, T, w.hist);
        PR_LAUNCHED("radix histogram");
        PR_TRY(scan_exclusive(w.hist, w.scanned, kRadixDigits * T, w.scan_ws, stream));
        if (p == 0)
            k_radix_scatter<MODE, false><<<dim3((unsigned)T), kBlock, 0, stream>>>(
                in, shift, T, w.scanned, kout, nullptr);
        else
            k_radix_scatter<kFromPairs, false><<<dim3((unsigned)T), kBlock, 0, stream>>>(
                in, shift, T, w.scanned, kout, nullptr);
        PR_LAUNCHED("radix scatter");
        in.keys = kout;
        *keys_sorted = kout;
    }
    return PR_OK;
}

}  // namespace pr
