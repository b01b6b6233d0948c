// Many tiny networks for gfx950 ("KiloNeRF: Speeding up Neural Radiance
// Fields with Thousands of Tiny MLPs", abstract: the scene is divided among
// thousands of small networks, with further optimisations such as skipping
// empty space and stopping rays early).
//
// One render pass runs as a pipeline of small kernels, with no host
// synchronisation:
//   count     one wave per ray: stratified samples, box and occupancy test,
//             live-sample mask and number of live samples per ray
//   scan      exclusive prefix sum of the counts (ray start offsets)
//   compact   32 rays per workgroup, one thread per live sample: live
//             samples written in (ray, sample) order with their cell id and
//             their rank among the workgroup's samples of that cell
//   cells     one workgroup: per-cell start offsets
//   scatter   live samples into per-cell buckets, as (point, entry, view
//             direction) records (bucket order within a cell is arbitrary:
//             each sample is its own matrix column and writes only its own
//             entry)
//   mlp       one workgroup per cell: the cell's network copied into LDS
//             once, then tiles of 64 (bf16) or 32 (f32) of its samples
//   composite 16 lanes per ray over its live samples in order (dead ones
//             change nothing), stop at the first with transmittance below term_T
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "mlp.hpp"
#include "raysteps.hpp"

namespace nerf {

constexpr int kScanBlock = kKiloScanBlock;

// ---------------------------------------------------------------------------
// Scans
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
    const int l = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t o = __shfl_up(v, off, kWave);
        if (l >= off) v += o;
    }
    return v;
}

// Exclusive scan of one value per thread over the workgroup (blockDim.x a
// multiple of 64, at most 1024).  lds needs 17 entries.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* lds, uint32_t& total) {
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave, nw = blockDim.x / kWave;
    const uint32_t incl = wave_incl_scan_u32(v);
    if (lane == kWave - 1) lds[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const uint32_t t = lane < nw ? lds[lane] : 0u;
        const uint32_t ti = wave_incl_scan_u32(t);
        if (lane < nw) lds[lane] = ti - t;
        if (lane == nw - 1) lds[16] = ti;
    }
    __syncthreads();
    const uint32_t res = lds[wave] + incl - v;
    total = lds[16];
    __syncthreads();
    return res;
}

__global__ void __launch_bounds__(256) k_scan_local(const uint32_t* __restrict__ in, uint32_t* __restrict__ out,
                                                    int64_t n, uint32_t* __restrict__ block_sums) {
    __shared__ uint32_t lds[17];
    const int64_t base = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * 4;
    uint32_t v[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = base + j < n ? in[base + j] : 0u;
        s += v[j];
    }
    uint32_t total;
    uint32_t run = block_excl_scan(s, lds, total);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (base + j < n) out[base + j] = run;
        run += v[j];
    }
    if (threadIdx.x == 0) block_sums[blockIdx.x] = total;
}

// One workgroup: exclusive scan of the block sums in place; entry nb = total.
__global__ void __launch_bounds__(1024) k_scan_blocks(uint32_t* __restrict__ bs, int64_t nb) {
    __shared__ uint32_t lds[17];
    uint32_t carry = 0;
    for (int64_t b0 = 0; b0 < nb; b0 += blockDim.x) {
        const int64_t i = b0 + threadIdx.x;
        const uint32_t v = i < nb ? bs[i] : 0u;
        uint32_t tot;
        const uint32_t ex = block_excl_scan(v, lds, tot);
        if (i < nb) bs[i] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) bs[nb] = carry;
}

__global__ void __launch_bounds__(256) k_scan_add(uint32_t* __restrict__ out, int64_t n,
                                                  const uint32_t* __restrict__ bs, int64_t nb) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] += bs[i / kScanBlock];
    if (i == n) out[n] = bs[nb];
}

__global__ void __launch_bounds__(256) k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// Samples and their classification
// ---------------------------------------------------------------------------
struct RayIn {
    float o[3], d[3], near, far;
};

__device__ __forceinline__ RayIn load_ray(const RenderArgs& a, int64_t r) {
    RayIn R;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        R.o[k] = a.ro[3 * r + k];
        R.d[k] = a.rd[3 * r + k];
    }
    R.near = a.tn[r];
    R.far = a.tf[r];
    return R;
}

// Depth of sample i of ray r (global counter ray_offset + r).
__device__ __forceinline__ float sample_z(const RenderArgs& a, const RayIn& R, int64_t r, int i) {
    const float u = a.jitter ? philox_uniform(a.seed, a.ray_offset + (uint64_t)r, (uint32_t)i, kStreamJitter) : 0.5f;
    return stratified_z(R.near, R.far, i, a.n_coarse, u);
}

// Sample i of ray r: z and the point.
__device__ __forceinline__ float sample_point(const RenderArgs& a, const RayIn& R, int64_t r, int i, float (&x)[3]) {
    const float z = sample_z(a, R, r, i);
#pragma unroll
    for (int k = 0; k < 3; ++k) x[k] = __fadd_rn(R.o[k], __fmul_rn(z, R.d[k]));
    return z;
}

// Live = inside the closed box and in an occupied voxel; also the cell id.
// Coordinates are floor((x - lo) * scale) of rounded float32 operations,
// clamped to the grid; ids are x-major.
__device__ __forceinline__ bool classify(const KiloArgs& k, const float (&x)[3], int& cell) {
    bool inside = true;
    int v[3], c[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        inside = inside && (x[a] >= k.lo) && (x[a] <= k.hi);
        const float t = __fsub_rn(x[a], k.lo);
        v[a] = grid_coord(t, k.vscale, k.occ_res);
        c[a] = grid_coord(t, k.cscale, k.cell_res);
    }
    // 64-bit: (occ_res)^3 passes 2^32 from occ_res = 1626 on
    const uint64_t res = (uint64_t)k.occ_res;
    const uint64_t vox = ((uint64_t)v[0] * res + (uint64_t)v[1]) * res + (uint64_t)v[2];
    cell = (c[0] * k.cell_res + c[1]) * k.cell_res + c[2];
    NERF_DCHECK((vox >> 5) < (res * res * res + 31u) / 32u, kCheckVoxel);
    NERF_DCHECK(cell >= 0 && cell < k.cell_res * k.cell_res * k.cell_res, kCheckCell);
    const bool occ = (k.occ[vox >> 5] >> (uint32_t)(vox & 31u)) & 1u;
    return inside && occ;
}

// The cell id alone (the same arithmetic as classify).
__device__ __forceinline__ int cell_of(const KiloArgs& k, const float (&x)[3]) {
    int c[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) c[a] = grid_coord(__fsub_rn(x[a], k.lo), k.cscale, k.cell_res);
    return (c[0] * k.cell_res + c[1]) * k.cell_res + c[2];
}

// Live-sample list of one ray from its mask words (bit i = sample i live):
// the sample indices in order, written to the wave's idx[]; returns their
// number.
__device__ __forceinline__ int live_list(const unsigned long long* mask, int words, int* idx) {
    const int lane = lane_id();
    const unsigned long long below = (1ull << lane) - 1ull;
    int c = 0;
    for (int w = 0; w < words; ++w) {
        const unsigned long long mw = mask[w];
        if ((mw >> lane) & 1ull) idx[c + __popcll(mw & below)] = kWave * w + lane;
        c += __popcll(mw);
    }
    wave_lds_sync();
    return c;
}

__global__ void __launch_bounds__(256) k_kilo_count(RenderArgs a, KiloArgs k) {
    const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (r >= a.n_rays) return;
    const RayIn R = load_ray(a, r);
    const int lane = lane_id();
    uint32_t cnt = 0;
    for (int base = 0; base < a.n_coarse; base += kWave) {
        const int i = base + lane;
        bool live = false;
        if (i < a.n_coarse) {
            float x[3];
            sample_point(a, R, r, i, x);
            int cell;
            live = classify(k, x, cell);
        }
        const unsigned long long m = __ballot(live);
        if (lane == 0) k.live_mask[r * k.mask_words + base / kWave] = m;
        cnt += __popcll(m);
    }
    if (lane == 0) k.live_count[r] = cnt;
}

constexpr int kKiloMaxSamples = 256;

// Compact: a workgroup takes kCompactRays consecutive rays, whose live
// samples are the contiguous entries [ray_start[r0], ray_start[r1]).  Each
// wave first lists the live samples of its rays into LDS (ray, sample), in
// order; then every thread takes one entry: its point, its cell, and its
// rank among the workgroup's samples of that cell, from an LDS hash table
// of per-cell counters (one LDS atomic per sample).  Each used table entry
// then takes one device-scope atomic for its base in the cell's bucket, and
// a last pass turns (entry, local rank) into bucket slots.  A sample that
// finds the table full takes its global slot directly (flagged in bit 31).
constexpr int kCompactRays = 32;
constexpr int kCellTable = 1024;  // power of two
constexpr uint32_t kSlotFinal = 0x80000000u;

__global__ void __launch_bounds__(256) k_kilo_compact(RenderArgs a, KiloArgs k) {
    __shared__ uint16_t ents[kCompactRays * kKiloMaxSamples];  // (ray - r0) << 8 | sample
    __shared__ int keys[kCellTable];
    __shared__ uint32_t counts[kCellTable];
    for (int i = threadIdx.x; i < kCellTable; i += blockDim.x) {
        keys[i] = -1;
        counts[i] = 0u;
    }
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const unsigned long long below = (1ull << lane) - 1ull;
    const int64_t r0 = (int64_t)blockIdx.x * kCompactRays;
    const int64_t r1 = r0 + kCompactRays < a.n_rays ? r0 + kCompactRays : a.n_rays;
    const uint32_t e0 = k.ray_start[r0], e1 = k.ray_start[r1];
    for (int j = 0; j < kCompactRays / 4; ++j) {
        const int64_t r = r0 + wave * (kCompactRays / 4) + j;
        if (r >= r1) break;
        const unsigned long long* mask = k.live_mask + r * k.mask_words;
        uint32_t c = k.ray_start[r] - e0;
        for (int w = 0; w < k.mask_words; ++w) {
            const unsigned long long mw = mask[w];
            NERF_DCHECK(!((mw >> lane) & 1ull) || c + __popcll(mw & below) < kCompactRays * kKiloMaxSamples,
                        kCheckCompactLds);
            if ((mw >> lane) & 1ull)
                ents[c + __popcll(mw & below)] = (uint16_t)(((uint32_t)(r - r0) << 8) | (uint32_t)(kWave * w + lane));
            c += (uint32_t)__popcll(mw);
        }
    }
    __syncthreads();
    for (uint32_t q = threadIdx.x; q < e1 - e0; q += blockDim.x) {
        const uint32_t pk = ents[q];
        const int64_t r = r0 + (pk >> 8);
        const int i = (int)(pk & 0xFFu);
        const RayIn R = load_ray(a, r);
        float x[3];
        sample_point(a, R, r, i, x);
        const int cell = cell_of(k, x);
        uint32_t slot = 0;
        int h = (int)(((uint32_t)cell * 2654435761u) >> 22) & (kCellTable - 1);
        int probes = 0;
        for (; probes < kCellTable; ++probes, h = (h + 1) & (kCellTable - 1)) {
            const int prev = atomicCAS(&keys[h], -1, cell);
            if (prev == -1 || prev == cell) break;
        }
        if (probes < kCellTable)
            slot = ((uint32_t)h << 20) | atomicAdd(&counts[h], 1u);
        else
            slot = kSlotFinal | atomicAdd(&k.cell_count[cell], 1u);
        const uint32_t e = e0 + q;
        NERF_DCHECK((uint64_t)e < (uint64_t)a.n_rays * (uint64_t)a.n_coarse, kCheckLiveEntry);
        k.ent_ray[e] = (uint32_t)r;
        k.ent_meta[e] = ((uint32_t)i << 16) | (uint32_t)cell;
        k.ent_slot[e] = slot;
    }
    __syncthreads();
    // one device-scope atomic per used table entry: its base in the bucket
    for (int h = threadIdx.x; h < kCellTable; h += blockDim.x) {
        const int c = keys[h];
        if (c >= 0) counts[h] = atomicAdd(&k.cell_count[c], counts[h]);
    }
    __syncthreads();
    for (uint32_t e = e0 + threadIdx.x; e < e1; e += blockDim.x) {
        const uint32_t t = k.ent_slot[e];
        k.ent_slot[e] = (t & kSlotFinal) ? (t & ~kSlotFinal) : counts[t >> 20] + (t & 0xFFFFFu);
    }
}

// One workgroup of 1024 threads: cell start offsets (exclusive scan of the
// per-cell counts; entry n_cells is the total).
__global__ void __launch_bounds__(1024) k_kilo_cells(KiloArgs k, int n_cells) {
    __shared__ uint32_t lds[17];
    uint32_t carry = 0;
    for (int c0 = 0; c0 < n_cells; c0 += blockDim.x) {
        const int c = c0 + threadIdx.x;
        const uint32_t cnt = c < n_cells ? k.cell_count[c] : 0u;
        uint32_t tot;
        const uint32_t ex = block_excl_scan(cnt, lds, tot);
        if (c < n_cells) k.cell_start[c] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) k.cell_start[n_cells] = carry;
}

// Grid-wide: live samples into their cells' buckets.  A bucket slot holds
// what the cell network needs, so that a tile's inputs are one contiguous
// read: (x, y, z, entry index) and the ray's unit direction.
__global__ void __launch_bounds__(256) k_kilo_scatter(RenderArgs a, KiloArgs k) {
    const uint32_t total = k.ray_start[a.n_rays];
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const uint32_t meta = k.ent_meta[e], r = k.ent_ray[e];
        const RayIn R = load_ray(a, r);
        float x[3];
        sample_point(a, R, r, (int)(meta >> 16), x);
        const float dn = sqrtf(R.d[0] * R.d[0] + R.d[1] * R.d[1] + R.d[2] * R.d[2]);
        NERF_DCHECK((uint64_t)k.cell_start[meta & 0xFFFFu] + k.ent_slot[e] < (uint64_t)a.n_rays * (uint64_t)a.n_coarse,
                    kCheckLiveEntry);
        f32x4* slot = reinterpret_cast<f32x4*>(k.bucket) + 2 * (size_t)(k.cell_start[meta & 0xFFFFu] + k.ent_slot[e]);
        slot[0] = f32x4{x[0], x[1], x[2], __uint_as_float(e)};
        slot[1] = f32x4{R.d[0] / dn, R.d[1] / dn, R.d[2] / dn, 0.0f};
    }
}

// A network held in LDS for the whole workgroup: the weight tiles are read
// with the same look-ahead as a stream from global memory.
template <class T, int KIND, int LOOK = 3>
struct LdsResident {
    using Op = typename T::Op;
    static constexpr int TB = tile_bytes(T::prec);
    static constexpr int NT = (int)(net_tiles_bytes(KIND, T::prec) / TB);
    const NERF_AS_LDS char* base;  // this lane's bytes of tile 0
    Op buf[LOOK];
    __device__ __forceinline__ LdsResident(const NERF_AS_LDS char* tiles, int lane)
        : base(tiles + lane * (int)sizeof(Op)) {}
    template <int TILE>
    __device__ __forceinline__ Op read() const {
        return *reinterpret_cast<const NERF_AS_LDS Op*>(base + TILE * TB);
    }
    __device__ __forceinline__ void begin() {
        static_for<0, LOOK>([&](auto t) {
            if constexpr (t.value < NT) buf[t.value] = read<t.value>();
        });
    }
    template <int TILE>
    __device__ __forceinline__ Op get() {
        const Op cur = buf[TILE % LOOK];
        if constexpr (TILE + LOOK < NT) buf[TILE % LOOK] = read<TILE + LOOK>();
        return cur;
    }
};

// One workgroup per cell: the cell's packed network (tiles and biases) is
// copied into LDS once, then the four waves take the cell's tiles of 32*SB
// bucketed samples in turn.
template <class T>
__global__ void __launch_bounds__(256) k_kilo_mlp(RenderArgs a, KiloArgs k) {
    constexpr int K = NET_CELL_2x32;
    constexpr int SB = T::SB;
    constexpr int ES = seg_steps(net_layers(K)[0].s0, T::prec);
    constexpr int DS = seg_steps(net_layers(K)[4].s1, T::prec);
    constexpr int NET_BYTES = (int)net_packed_bytes(K, T::prec);
    static_assert(NET_BYTES % 16 == 0, "16-byte copies");
    __shared__ __attribute__((aligned(16))) char net[NET_BYTES];
    const uint32_t c = blockIdx.x;
    const uint32_t cs = k.cell_start[c], cnt = k.cell_start[c + 1] - cs;
    if (cnt == 0) return;
    const char* packed = (const char*)k.cells + (size_t)c * k.cell_stride;
    for (int o = threadIdx.x * 16; o < NET_BYTES; o += blockDim.x * 16)
        *reinterpret_cast<f32x4*>(net + o) = *reinterpret_cast<const f32x4*>(packed + o);
    __syncthreads();
    const NERF_AS_LDS char* lnet = (const NERF_AS_LDS char*)net;
    const NERF_AS_LDS float* bias = (const NERF_AS_LDS float*)(lnet + net_bias_offset(K, T::prec, 0));
    const int lane = lane_id();
    const uint32_t n_tiles = (cnt + 32 * SB - 1) / (32 * SB);
    const f32x4* slots = reinterpret_cast<const f32x4*>(k.bucket) + 2 * (size_t)cs;
    // a tile's bucket slots, read one tile ahead of their use
    auto fetch = [&](uint32_t t, f32x4 (&p)[SB], f32x4 (&q)[SB]) {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            const uint32_t j = t * 32 * SB + sb * 32 + (lane & 31);
            const uint32_t jj = j < cnt ? j : cnt - 1;
            p[sb] = slots[2 * jj];
            q[sb] = slots[2 * jj + 1];
        }
    };
    constexpr uint32_t kWaves = 256 / kWave;
    uint32_t t = threadIdx.x / kWave;
    f32x4 p[SB], q[SB];
    if (t < n_tiles) fetch(t, p, q);
    for (; t < n_tiles; t += kWaves) {
        f32x4 pn[SB], qn[SB];
        if (t + kWaves < n_tiles) fetch(t + kWaves, pn, qn);
        float x[SB][3], v[SB][3];
        uint32_t e[SB];
        bool valid[SB];
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            valid[sb] = t * 32 * SB + sb * 32 + (lane & 31) < cnt;
            e[sb] = __float_as_uint(p[sb][3]);
#pragma unroll
            for (int c3 = 0; c3 < 3; ++c3) {
                x[sb][c3] = p[sb][c3];
                v[sb][c3] = q[sb][c3];
            }
        }
        typename T::Op enc[ES][SB], denc[DS][SB];
        enc_operands<10>(enc, x, a.use_pi != 0, lane);
        enc_operands<4>(denc, v, a.use_pi != 0, lane);
        LdsResident<T, K> ws(lnet, lane);
        f32x16 sig[SB], rgb[SB];
        nerf_forward<T, K>(enc, denc, ws, bias, sig, rgb, lane);
        if (lane < 32) {
#pragma unroll
            for (int sb = 0; sb < SB; ++sb)
                if (valid[sb])
                    reinterpret_cast<f32x4*>(k.raw_live)[e[sb]] =
                        f32x4{rgb[sb][0], rgb[sb][1], rgb[sb][2], sig[sb][0]};
        }
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            p[sb] = pn[sb];
            q[sb] = qn[sb];
        }
    }
}

// Sixteen lanes per ray (four rays per wave), over its live samples only: a
// dead sample has density 0, so its weight is 0 and its survival factor
// 1 - 0 + 1e-10 rounds to 1 in float32 - skipping it changes no product.  A
// live sample's interval needs the depth of the next sample, live or not
// (recomputed from its counter).  Transmittance is a 16-lane product scan
// per chunk of live samples, carried across chunks.
constexpr int kRowLanes = 16;

__device__ __forceinline__ float row_scan_mul(float v, int j) {
#pragma unroll
    for (int off = 1; off < kRowLanes; off <<= 1) {
        const float o = __shfl_up(v, off, kRowLanes);
        if (j >= off) v *= o;
    }
    return v;
}

__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
    for (int off = kRowLanes / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kRowLanes);
    return v;
}

__global__ void __launch_bounds__(256) k_kilo_composite(RenderArgs a, KiloArgs k) {
    constexpr int RAYS = 256 / kRowLanes;
    __shared__ uint8_t lists[RAYS][kKiloMaxSamples];
    const int lane = lane_id();
    const int row = lane / kRowLanes, j = lane % kRowLanes;
    const int slot = (int)(threadIdx.x / kRowLanes);
    const int64_t r_raw = (int64_t)blockIdx.x * RAYS + slot;
    const bool ray_ok = r_raw < a.n_rays;
    const int64_t r = ray_ok ? r_raw : a.n_rays - 1;  // a row past the last ray repeats it and stores nothing
    const RayIn R = load_ray(a, r);
    const int N = a.n_coarse;
    const float dn = sqrtf(R.d[0] * R.d[0] + R.d[1] * R.d[1] + R.d[2] * R.d[2]);
    if (a.dbg_z && ray_ok)
        for (int i = j; i < N; i += kRowLanes) a.dbg_z[r * N + i] = sample_z(a, R, r, i);
    // the ray's live samples, in order: lane j of the row takes bits 4j..4j+3 of each mask word
    uint8_t* list = lists[slot];
    const unsigned long long* mask = k.live_mask + r * k.mask_words;
    int nlive = 0;
    for (int w = 0; w < k.mask_words; ++w) {
        const unsigned long long mw = mask[w];
        const uint32_t sub = (uint32_t)(mw >> (4 * j)) & 0xFu;
        int at = nlive + __popcll(mw & ((1ull << (4 * j)) - 1ull));
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if ((sub >> b) & 1u) list[at++] = (uint8_t)(kWave * w + 4 * j + b);
        nlive += __popcll(mw);
    }
    wave_lds_sync();
    const f32x4* raw = reinterpret_cast<const f32x4*>(k.raw_live) + k.ray_start[r];
    float carry = 1.0f, sr = 0.f, sg = 0.f, sbl = 0.f, sd = 0.f, sa = 0.f;
    bool stopped = false;
    for (int base = 0; __ballot(base < nlive && !stopped); base += kRowLanes) {
        const int q = base + j;
        const bool valid = q < nlive && !stopped;
        float alpha = 0.f, zi = 0.f;
        f32x4 rw = {0.f, 0.f, 0.f, 0.f};
        if (valid) {
            const int i = list[q];
            zi = sample_z(a, R, r, i);
            const float delta = (i + 1 < N) ? (sample_z(a, R, r, i + 1) - zi) * dn : 1e10f * dn;
            rw = raw[q];
            alpha = 1.0f - expf(-fmaxf(rw[3], 0.0f) * delta);
        }
        const float surv = valid ? (1.0f - alpha + 1e-10f) : 1.0f;
        const float incl = row_scan_mul(surv, j);
        float excl = __shfl_up(incl, 1, kRowLanes);
        if (j == 0) excl = 1.0f;
        const float T = carry * excl;
        bool stop_here = false;
        if (k.term_T > 0.0f) {
            // the first live sample (in order) with T < term_T and all later ones are dropped
            const unsigned long long m = __ballot(valid && T < k.term_T);
            const uint32_t mrow = (uint32_t)(m >> (kRowLanes * row)) & 0xFFFFu;
            const int first = mrow ? __builtin_ctz(mrow) : kRowLanes;
            stop_here = j >= first;
            if (mrow) stopped = true;
        }
        const float w = (valid && !stop_here) ? T * alpha : 0.0f;
        sa += w;
        sd += w * zi;
        sr += w * sigmoidf_(rw[0]);
        sg += w * sigmoidf_(rw[1]);
        sbl += w * sigmoidf_(rw[2]);
        carry *= __shfl(incl, kRowLanes - 1, kRowLanes);
    }
    sr = row_sum(sr);
    sg = row_sum(sg);
    sbl = row_sum(sbl);
    sd = row_sum(sd);
    sa = row_sum(sa);
    if (j == 0 && ray_ok) {
        const float bg = a.white ? 1.0f - sa : 0.0f;
        a.rgb[3 * r] = sr + bg;
        a.rgb[3 * r + 1] = sg + bg;
        a.rgb[3 * r + 2] = sbl + bg;
        a.depth[r] = sd;
        a.acc[r] = sa;
    }
}

// Number of live samples of this chunk, written (first chunk) or added.
__global__ void k_kilo_n_live(const uint32_t* __restrict__ ray_start, int64_t n_rays, int64_t* out, int add) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *out = (add ? *out : 0) + (int64_t)ray_start[n_rays];
}

// ---------------------------------------------------------------------------
// Workspace and launch
// ---------------------------------------------------------------------------
void launch_render_kilo(int bf16, const RenderArgs& a, const KiloArgs& k, int add_n_live, hipStream_t s) {
    const int64_t n = a.n_rays;
    const int n_cells = k.cell_res * k.cell_res * k.cell_res;
    const dim3 rays4((unsigned)((n + 3) / 4));
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n_cells + 255) / 256)), dim3(256), 0, s, k.cell_count,
                       (int64_t)n_cells, 0u);
    hipLaunchKernelGGL(k_kilo_count, rays4, dim3(256), 0, s, a, k);
    const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
    hipLaunchKernelGGL(k_scan_local, dim3((unsigned)nb), dim3(256), 0, s, k.live_count, k.ray_start, n, k.block_sums);
    hipLaunchKernelGGL(k_scan_blocks, dim3(1), dim3(1024), 0, s, k.block_sums, nb);
    hipLaunchKernelGGL(k_scan_add, dim3((unsigned)((n + 1 + 255) / 256)), dim3(256), 0, s, k.ray_start, n,
                       k.block_sums, nb);
    hipLaunchKernelGGL(k_kilo_compact, dim3((unsigned)((n + kCompactRays - 1) / kCompactRays)), dim3(256), 0, s, a, k);
    hipLaunchKernelGGL(k_kilo_cells, dim3(1), dim3(1024), 0, s, k, n_cells);
    hipLaunchKernelGGL(k_kilo_scatter, dim3(2048), dim3(256), 0, s, a, k);
    if (bf16)
        hipLaunchKernelGGL(k_kilo_mlp<TBF16>, dim3((unsigned)n_cells), dim3(256), 0, s, a, k);
    else
        hipLaunchKernelGGL(k_kilo_mlp<TF32>, dim3((unsigned)n_cells), dim3(256), 0, s, a, k);
    hipLaunchKernelGGL(k_kilo_composite, dim3((unsigned)((n + 15) / 16)), dim3(256), 0, s, a, k);
    if (k.dbg_n_live)
        hipLaunchKernelGGL(k_kilo_n_live, dim3(1), dim3(64), 0, s, k.ray_start, n, k.dbg_n_live, add_n_live);
}

}  // namespace nerf
