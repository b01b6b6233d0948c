/*
 * nerf_mi355x.h - C ABI of libnerf_mi355x.so, the NeRF forward-render hot
 * path for AMD Instinct MI355X (gfx950).
 *
 * What the calls compute is defined by the blog post "Spatial Intelligence -
 * Part 1: NeRF" (Section 1 Theory and Section 2 Code), the notebook
 * "Instant-NGP - Visual Experiments (a 2D multiresolution hash grid)" (its
 * shared toolkit, generalised here to 3D) and the abstract of "KiloNeRF:
 * Speeding up Neural Radiance Fields with Thousands of Tiny MLPs".
 *
 * Conventions shared by every call
 *  - Pointers documented as "device" are device memory of the current HIP
 *    device, owned by the caller, contiguous, row-major, 16-byte aligned.
 *    Pointers documented as "host" are ordinary host memory.  The library
 *    keeps no pointer after a call returns (it is stateless apart from
 *    immutable kernel handles).
 *  - All floating tensors are float32 unless stated.  Rays are in pixel
 *    order, ray index = row * W + column.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call that
 *    takes a stream only enqueues work on it and returns; inputs must stay
 *    unchanged until the stream reaches the work.  Calls are thread-safe and
 *    may run concurrently on different streams.
 *  - Arguments are validated before anything is enqueued.  A call returns
 *    NERF_OK, or an error status with nothing enqueued, and the reason is
 *    kept in a thread-local string returned by nerf_last_error().  n == 0
 *    (no rays, no points) returns NERF_OK without launching.  HIP launch
 *    errors map to NERF_ERR_HIP.  Faults inside a kernel surface at the
 *    caller's next synchronisation.  NaN and Inf inputs are not checked;
 *    they propagate.  No C++ exception crosses this interface.
 */
#ifndef NERF_MI355X_H
#define NERF_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NERF_ABI_VERSION 2

typedef enum {
    NERF_OK = 0,
    NERF_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad enum, misalignment */
    NERF_ERR_UNSUPPORTED = 2,      /* valid but not built: network shape, sample count, ... */
    NERF_ERR_WORKSPACE = 3,        /* workspace missing or too small */
    NERF_ERR_HIP = 4               /* a HIP runtime call failed */
} nerf_status;

typedef enum { NERF_F32 = 0, NERF_BF16 = 1 } nerf_dtype;

/* Network families the library is built for.  Each kind fixes the layer
 * shapes; the matrix-engine input precision is chosen by nerf_mlp_desc.dtype.
 *
 * NERF_NET_8x256: the page's network ("4. The NeRF network"): 8 ReLU layers
 *   of width 256 on the position encoding (63 = 3 + 6*10), the encoding
 *   concatenated after the hidden state of layer index 4 (layer 5 sees 319
 *   inputs), density head 256 -> 1, linear feature layer 256 -> 256,
 *   direction layer [feature, direction encoding (27 = 3 + 6*4)] -> 128 ReLU,
 *   rgb head 128 -> 3.
 * NERF_NET_4x64: the same family, 4 layers of width 64, no skip, position
 *   encoding of 6 frequencies (39), direction layer width 32.
 * NERF_NET_CELL_2x32: the same family, 2 layers of width 32, no skip, position
 *   encoding 63, direction layer width 16 (one tiny network per cell).
 * NERF_NET_HASH_FIELD: hash-grid field: 32 grid features -> 64 -> 64 (ReLU),
 *   density head 64 -> 1, linear feature layer 64 -> 64, colour net
 *   [feature, 16 spherical harmonics] -> 64 -> 64 (ReLU), rgb head 64 -> 3.
 *
 * Every network outputs raw = (rgb_raw[3], sigma_raw) per sample, without
 * activations; the compositor applies sigmoid and ReLU. */
typedef enum {
    NERF_NET_8x256 = 1,
    NERF_NET_4x64 = 2,
    NERF_NET_CELL_2x32 = 3,
    NERF_NET_HASH_FIELD = 4
} nerf_net_kind;

typedef struct {
    int32_t kind;  /* nerf_net_kind */
    int32_t dtype; /* nerf_dtype: NERF_BF16 rounds weights and layer inputs to
                      bfloat16 (round to nearest even) and accumulates in
                      float32; NERF_F32 keeps float32 throughout */
} nerf_mlp_desc;

typedef enum { NERF_MODE_NERF = 0, NERF_MODE_HASH = 1, NERF_MODE_KILO = 2 } nerf_render_mode;

/* Pinhole camera.  The page's camera ("2. Ray generation") is fx = fy =
 * focal, cx = W/2, cy = H/2, no half-pixel shift. */
typedef struct {
    int32_t W, H;
    float fx, fy, cx, cy;
} nerf_intrinsics;

/* Multiresolution grid over [0,1]^dim ("Instant-NGP - Visual Experiments",
 * shared toolkit ``HashGrid2D``, and its generalisation to 3D).  Filled by
 * nerf_hashgrid_init(); `tables` is set by the caller; `level_mask` may be
 * changed by the caller. */
#define NERF_HASH_MAX_LEVELS 16
typedef struct {
    int32_t n_levels;                     /* L <= 16 */
    int32_t n_feat;                       /* features per entry; must be 2 */
    uint32_t table_size;                  /* T, a power of two */
    int32_t res[NERF_HASH_MAX_LEVELS];    /* N_l */
    int32_t direct[NERF_HASH_MAX_LEVELS]; /* 1: (N_l+1)^3 <= T, direct index */
    uint32_t size[NERF_HASH_MAX_LEVELS];  /* entries of level l: min(T, (N_l+1)^3) */
    uint64_t offset[NERF_HASH_MAX_LEVELS];/* first entry of level l in `tables` */
    uint64_t total_entries;               /* sum of size[] */
    const void* tables;                   /* device, float16 [total_entries][n_feat], 8-byte aligned;
                                             read in aligned 8-byte words, so readable up to
                                             total_entries rounded up to an even count (any
                                             allocation rounded to 8 bytes is); at most 2^28 entries */
    int32_t dim;                          /* 2 or 3 */
    float level_mask[NERF_HASH_MAX_LEVELS];/* level l's features are multiplied by level_mask[l]
                                             (the toolkit's level_mask: coarse-to-fine evaluation);
                                             nerf_encode_hashgrid does not look up a level whose
                                             mask is 0; init: 1 */
} nerf_hashgrid;

/* Weights handed to nerf_render.  Packed networks come from nerf_pack_mlp and
 * live in device memory. */
typedef struct {
    nerf_mlp_desc net;          /* the network kind/precision of every packed net below */
    const void* coarse;         /* NERF: first-pass network; HASH: the field network */
    const void* fine;           /* NERF with n_fine > 0: second-pass network */
    const void* cells;          /* KILO: n_cells packed networks back to back,
                                   nerf_mlp_packed_bytes(&net) apart */
    int32_t n_cells;            /* KILO: cell_res^3 */
    const nerf_hashgrid* grid;  /* HASH: host struct, tables on the device */
} nerf_weights;

typedef struct {
    int32_t mode;          /* nerf_render_mode */
    int32_t n_coarse;      /* samples per ray of the first pass: 1..256 */
    int32_t n_fine;        /* NERF: inverse-CDF samples, 0 = first pass only;
                              n_coarse >= 3 and n_coarse + n_fine <= 256 */
    int32_t use_pi;        /* 1: sin(2^k pi x) (theory, "4.1 Positional
                              encoding"); 0: sin(2^k x) (the page's code) */
    int32_t white_bkgd;    /* add 1 - acc to rgb ("5. Volume rendering in code") */
    int32_t jitter;        /* 1: one uniform per stratum; 0: stratum centres */
    uint64_t seed;         /* Philox key for jitter and inverse-CDF uniforms */
    uint64_t ray_offset;   /* global index of ray 0: the counter of ray r is ray_offset + r */
    int64_t chunk;         /* rays per launch (0: all); results do not depend on it */
    float term_T;          /* drop sample i and later once T_i < term_T (0: never); NERF/HASH
                              also stop evaluating a ray's samples there */
    float box_lo, box_hi;  /* scene box [lo,hi]^3 of the occupancy grid (HASH also maps it to [0,1]^3) */
    int32_t occ_res;       /* occupancy grid resolution per axis (128) */
    int32_t cell_res;      /* KILO: cells per axis (16) */
    const uint32_t* occ;   /* device bitset, bit v%32 of word v/32 for voxel
                              v = (vx*res + vy)*res + vz, vx = clamp(floor((x-lo)*res/(hi-lo)));
                              a sample outside the box or in an empty voxel has density 0 and is
                              not evaluated.  Required in KILO mode; NULL in NERF/HASH: no skipping */
    void* workspace;       /* device scratch (KILO); NULL: the call allocates
                              it stream-ordered and frees it after the work */
    size_t workspace_bytes;
    float* dbg_z;          /* optional device [n_rays, n_coarse + n_fine]: samples of the last pass */
    float* dbg_w_coarse;   /* optional device [n_rays, n_coarse]: first-pass weights */
    int64_t* dbg_n_live;   /* optional device int64[1]: live samples (inside the box and
                              occupied; every sample without a grid), over both passes */
} nerf_render_cfg;

/* ---------------------------------------------------------------------- */
/* Library information                                                    */
/* ---------------------------------------------------------------------- */

int nerf_abi_version(void);

/* Index checks of the kernels.  In a library built with -DNERF_CHECK
 * (libnerf_mi355x_checked.so) the kernels record failed index-range checks
 * (hash-grid corner indices, ray-sample and merged-sample positions,
 * inverse-CDF bins, occupancy words, cell ids, live-list entries and bucket
 * slots) and failed input preconditions as bits of a flag word instead of
 * faulting.  This call waits for the
 * device, returns the bits set since the previous call (0: none) and clears
 * them; a library built without the checks returns -1.  Bits: 0 hash-grid
 * corner index outside its level's table, 1 sample index outside a ray's
 * sample arrays, 2 inverse-CDF bin outside 1 .. n_coarse - 2, 3 merged
 * sample position outside the merged array, 4 occupancy word outside the
 * bitset, 5 cell id outside the cell grid, 6 live-list entry or bucket slot
 * outside the workspace, 7 compaction entry outside a workgroup's LDS list,
 * 8 an inverse-CDF weight outside nerf_sample_pdf's precondition (finite, in
 * [0, 100]); all bits set: the flags could not be read. */
int64_t nerf_check_flags(void);
const char* nerf_status_str(nerf_status s);
/* Thread-local text of the last error on this thread ("" if none). */
const char* nerf_last_error(void);

/* ---------------------------------------------------------------------- */
/* Host helpers                                                           */
/* ---------------------------------------------------------------------- */

/* Fills res/direct/size/offset/total_entries of `g` (host) for a grid over
 * [0,1]^dim with L levels of resolutions N_l = round(n_min * b^l),
 * b = exp((ln n_max - ln n_min)/(L-1)), direct indexing where
 * (N_l+1)^dim <= T ("Instant-NGP - Visual Experiments", shared toolkit;
 * Experiments 1 and 4).  n_feat is set to 2, tables to NULL, every
 * level_mask to 1.  Errors: dim not 2 or 3, L outside 2..16, T not a power
 * of two, n_min < 1, n_max < n_min. */
nerf_status nerf_hashgrid_init(nerf_hashgrid* g, int dim, int n_levels, uint32_t table_size, int n_min, int n_max);

/* Bytes of one packed network of this description (0 if unsupported). */
size_t nerf_mlp_packed_bytes(const nerf_mlp_desc* net);

/* Packs float32 weights (host) into the device-ready layout (written to host
 * memory `dst`, which the caller copies to the device).  `tensors` lists
 * row-major [out, in] weight matrices and [out] biases in forward order:
 *   NeRF kinds: W_0, b_0, ..., W_{D-1}, b_{D-1}, W_sigma, b_sigma,
 *               W_feature, b_feature, W_dir, b_dir, W_rgb, b_rgb
 *               (layer skip+1 has inputs [hidden, position encoding];
 *                W_dir has inputs [feature, direction encoding]);
 *   HASH_FIELD: W_d0, b_d0, W_d1, b_d1, W_sigma, b_sigma, W_feature,
 *               b_feature, W_c0, b_c0, W_c1, b_c1, W_rgb, b_rgb
 *               (W_c0 has inputs [feature, 16 harmonics]).
 * Encoding columns follow the frequency-major layout of nerf_encode_freq.
 * For NERF_BF16 the weights are rounded to bfloat16 here.
 * Errors: unsupported kind, wrong n_tensors, null pointers, dst too small. */
nerf_status nerf_pack_mlp(const nerf_mlp_desc* net, const float* const* tensors, int n_tensors,
                          void* dst, size_t dst_bytes);

/* ---------------------------------------------------------------------- */
/* Hot-path steps (device)                                                */
/* ---------------------------------------------------------------------- */

/* Rays of a pinhole camera ("Spatial Intelligence - Part 1: NeRF", Section 2
 * Code, 2. Ray generation).  pose: host float[12], row-major 3x4
 * camera-to-world [R | t].  For pixel (i = column, j = row):
 *   d_cam = ((i - cx)/fx, -((j - cy)/fy), -1),  d = R d_cam (not normalised),
 *   o = t,
 * each float32 operation rounded (no fused multiply-add; d_k is summed left
 * to right), so results are bit-reproducible.
 * rays_o, rays_d: device [W*H, 3].  Errors: null pointers, W or H < 1,
 * fx or fy == 0. */
nerf_status nerf_gen_rays(const float* pose, const nerf_intrinsics* K, float* rays_o, float* rays_d,
                          void* stream);

/* Stratified samples (Section 1 Theory, 3. Volume rendering; the page's
 * stratified_sample, read as one uniform draw per equal stratum):
 *   step = (far - near)/n;  z_i = near + step*(i + u_i)
 * as rounded float32 operations; u_i = Philox4x32-10 uniform of counter
 * (ray lo, i, ray hi, 0) under key seed, ray = ray_offset + r; u = 1/2 when
 * jitter == 0.  t_near, t_far: device [n_rays]; z: device [n_rays, n].
 * Errors: null pointers, n_rays < 0, n outside 1..256. */
nerf_status nerf_sample_stratified(const float* t_near, const float* t_far, int64_t n_rays, int n,
                                   uint64_t seed, uint64_t ray_offset, int jitter, float* z, void* stream);

/* Frequency encoding (Section 1 Theory, 4.1 Positional encoding):
 *   gamma(p) = (p, sin(2^0 pi p), cos(2^0 pi p), ..., sin(2^{L-1} pi p), cos(2^{L-1} pi p))
 * frequency-major: the input (if include_input), then per k the in_dim
 * sines followed by the in_dim cosines; use_pi = 0 drops pi.  x: device
 * [n, in_dim]; out: device [n, in_dim*(include_input + 2L)] of out_dtype
 * (NERF_F32, or NERF_BF16 rounded to nearest even).  Accuracy: sin/cos of
 * the exact argument 2^k x, within 2.4e-7 of the exact value.
 * Errors: null pointers, n < 0, in_dim outside 1..4, n_freq outside 0..16,
 * bad dtype. */
nerf_status nerf_encode_freq(const float* x, int64_t n, int in_dim, int n_freq, int include_input, int use_pi,
                             int out_dtype, void* out, void* stream);

/* 16 real spherical harmonics of degrees 0..3 (orthonormal, no
 * Condon-Shortley phase, ordered by degree then order -l..l) of unit
 * directions: the 16-wide direction encoding of the hash-grid field.
 * dirs: device [n, 3] (normalised inside); out: device [n, 16]. */
nerf_status nerf_encode_sh16(const float* dirs, int64_t n, float* out, void* stream);

/* Multiresolution hash-grid encoding ("Instant-NGP - Visual Experiments",
 * shared toolkit ``HashGrid2D.encode``, and its extension to 3D): per level
 * c = x*N_l (float32), c0 = floor(c), w = c - c0; for the 2^dim corners
 * (lexicographic, x most significant) corner coordinates clamped to [0,N_l];
 * index ix*(N+1) + iy (2D) or ((ix*(N+1)) + iy)*(N+1) + iz (3D) on direct
 * levels, else (ix ^ iy*2654435761) mod T (2D) or
 * (ix*1 ^ iy*2654435761 ^ iz*805459861) mod T (3D); feature = level_mask[l]
 * * sum over corners of prod(w or 1-w) * table[index]; levels concatenated
 * (level-major, then feature).  x: device [n, dim] (points outside the unit
 * cube use clamped corners); out: device [n, L*2]; idx_dbg: optional device
 * uint32 [n, L, 2^dim] corner indices (levels with mask 0 are not looked up
 * and their indices are not written).  Errors: null pointers, n < 0, grid
 * not initialised, null tables. */
nerf_status nerf_encode_hashgrid(const float* x, int64_t n, const nerf_hashgrid* g, float* out, uint32_t* idx_dbg,
                                 void* stream);

/* The radiance network on encoded inputs (Section 2 Code, 4. The NeRF
 * network, NeRF.forward; hash field for NERF_NET_HASH_FIELD).
 * packed: device, from nerf_pack_mlp.  enc_x: device [n, in_ch] (position
 * encoding 63/39 wide for NeRF kinds, 32 grid features for the hash field);
 * enc_v: device [ceil(n / samples_per_ray), dir_ch] per-ray direction
 * encoding (27 for NeRF kinds, 16 harmonics for the hash field); sample s
 * uses row s / samples_per_ray.  raw: device [n, 4] = (rgb_raw, sigma_raw).
 * Errors: unsupported desc, null pointers, n < 0, samples_per_ray < 1. */
nerf_status nerf_mlp(const nerf_mlp_desc* net, const void* packed, const float* enc_x, const float* enc_v,
                     int64_t n, int samples_per_ray, float* raw, void* stream);

/* Alpha compositing (Section 1 Theory, 3. Volume rendering; Section 2 Code,
 * 5. Volume rendering in code): delta_i = (z_{i+1} - z_i)|d|, last
 * 1e10|d|; alpha = 1 - exp(-relu(sigma) delta); T = exclusive product of
 * (1 - alpha + 1e-10); w = T alpha; rgb = sum w sigmoid(rgb_raw);
 * depth = sum w z; acc = sum w; rgb += 1 - acc if white_bkgd.
 * raw: device [n_rays, n, 4]; z: device [n_rays, n]; rays_d: device
 * [n_rays, 3]; rgb [n_rays, 3], depth, acc [n_rays]; weights optional device
 * [n_rays, n].  Errors: null pointers, n_rays < 0, n outside 1..4096. */
nerf_status nerf_composite(const float* raw, const float* z, const float* rays_d, int64_t n_rays, int n,
                           int white_bkgd, float* rgb, float* depth, float* acc, float* weights, void* stream);

/* Inverse-CDF resampling and merge (Section 1 Theory, 4.2 Hierarchical
 * volume sampling; Section 2 Code, 6. Hierarchical sampling, sample_pdf
 * called on midpoints(z) with weights[1:-1]): bins b_k = (z_k + z_{k+1})/2
 * (float32), w'_j = w_{j+1} + 1e-5 (float32), cdf = exact float64 running sum
 * of w' divided by its total (cdf_0 = 0, last = 1); u_m = Philox uniform of
 * counter (ray lo, m, ray hi, 1); idx = #{k: cdf_k <= u}; below/above =
 * idx-1/idx clamped; denom = max(cdf_above - cdf_below, 1e-5);
 * z = b_below + (u - cdf_below)/denom * (b_above - b_below) in float64
 * rounded once to float32.  Bins and samples are bit-reproducible.
 * z_coarse, w_coarse: device [n_rays, n_coarse]; outputs (each optional,
 * device): z_fine [n_rays, n_fine], bin_idx int32 [n_rays, n_fine],
 * z_merged [n_rays, n_coarse + n_fine] ascending.
 * Errors: null inputs, n_rays < 0, n_coarse < 3, n_fine < 1,
 * n_coarse + n_fine > 256. */
nerf_status nerf_sample_pdf(const float* z_coarse, const float* w_coarse, int64_t n_rays, int n_coarse,
                            int n_fine, uint64_t seed, uint64_t ray_offset, float* z_fine, int32_t* bin_idx,
                            float* z_merged, void* stream);

/* The whole forward render of each ray (Section 2 Code, 6. Hierarchical
 * sampling, render_rays; the hash-grid field; many tiny cell networks):
 *  NERF: stratified samples -> position/direction encoding -> coarse network
 *        -> compositing -> (n_fine > 0) inverse-CDF resampling, merge ->
 *        fine network on the merged samples -> compositing.
 *  HASH: stratified samples -> world box to unit cube -> hash-grid features,
 *        harmonics of the view direction -> field network -> compositing.
 *  NERF and HASH skip empty space when cfg.occ is set (Section 1 Theory,
 *  4.2: uniform samples waste compute on empty space): only live samples
 *  are evaluated, the others have density 0; with term_T > 0 a ray stops
 *  evaluating once its transmittance is below term_T, and compositing drops
 *  sample i and later once T_i < term_T.
 *  KILO: stratified samples -> occupancy and box test -> cell id -> cell
 *        network for occupied samples (density 0 elsewhere) -> compositing
 *        that stops at the first sample with T < term_T.
 * rays_o, rays_d: device [n_rays, 3]; t_near, t_far: device [n_rays];
 * rgb: device [n_rays, 3]; depth, acc: device [n_rays].  Nothing else is
 * written except the optional dbg_* outputs of cfg.
 * Errors: null pointers, mode/network mismatch, unsupported sample counts,
 * workspace too small (KILO). */
nerf_status nerf_render(const float* rays_o, const float* rays_d, const float* t_near, const float* t_far,
                        int64_t n_rays, const nerf_weights* w, const nerf_render_cfg* cfg, float* rgb, float* depth,
                        float* acc, void* stream);

/* One image per camera pose (Section 2 Code, 1. Overview: render_image and
 * the video of a pose sweep).  For frame f: the rays of pose f and camera K
 * (as nerf_gen_rays), t_near and t_far for every ray, then nerf_render with
 * cfg.ray_offset + f*W*H as the ray offset, so every pixel of every frame has
 * its own random-number counters.  poses: host [n_poses][12] row-major 3x4
 * camera-to-world; rgb: device [n_poses, H*W, 3]; depth, acc: device
 * [n_poses, H*W].  workspace: device, 16-byte aligned, at least 32*W*H bytes
 * (one frame's rays and near/far), or NULL: allocated stream-ordered and
 * freed after the work.  The debug outputs of cfg must be NULL.
 * Errors: as nerf_gen_rays and nerf_render; workspace too small. */
nerf_status nerf_render_poses(const float* poses, int n_poses, const nerf_intrinsics* K, float t_near, float t_far,
                              const nerf_weights* w, const nerf_render_cfg* cfg, void* workspace,
                              size_t workspace_bytes, float* rgb, float* depth, float* acc, void* stream);

/* Device workspace nerf_render needs for this configuration (0 for NERF and
 * HASH modes). */
size_t nerf_render_workspace_size(const nerf_render_cfg* cfg, int64_t n_rays);

/* ---------------------------------------------------------------------- */
/* Training step (device)                                                 */
/* ---------------------------------------------------------------------- */

/* Configuration of one training step of a NeRF-family network. */
typedef struct {
    nerf_mlp_desc net;     /* NERF_NET_8x256, NERF_NET_4x64 or NERF_NET_CELL_2x32; dtype: operand
                              precision of every matrix product, forward and backward
                              (NERF_BF16: bfloat16 operands, float32 accumulation) */
    int32_t n_samples;     /* stratified samples per ray: 1..256 */
    int32_t use_pi;        /* as nerf_render_cfg */
    int32_t white_bkgd;
    int32_t jitter;
    uint64_t seed;         /* Philox key of the stratified jitter (as nerf_sample_stratified) */
    uint64_t ray_offset;   /* global index of ray 0 */
    float lr, beta1, beta2, eps; /* Adam */
    const float* z;        /* optional device [n_rays, n_samples], ascending per ray: the sample
                              depths to use instead of stratified ones (the fine pass of the
                              page's training step: merged coarse and inverse-CDF samples, which
                              carry no gradient); NULL: stratified */
    float* weights;        /* optional device [n_rays, n_samples]: the compositing weights
                              w_i = T_i alpha_i of this pass (input to nerf_sample_pdf) */
} nerf_train_cfg;

/* Flat parameter count of a network kind: the weights and biases in the
 * order nerf_pack_mlp takes them, each row-major, back to back (0 if the
 * kind cannot be trained here). */
int64_t nerf_train_param_count(int kind);

/* Device workspace of nerf_train_step for n_rays rays (0 if unsupported). */
size_t nerf_train_workspace_size(const nerf_train_cfg* cfg, int64_t n_rays);

/* One training step ("Spatial Intelligence - Part 1: NeRF", Section 1
 * Theory, 5. Training; Section 2 Code, 7. Training loop, one network pass):
 * stratified samples (as nerf_sample_stratified), position and direction
 * encodings (as nerf_encode_freq), the network (as nerf_mlp), compositing
 * (as nerf_composite), loss = mean over rays and channels of
 * (rgb - target)^2, the gradient of the loss with respect to every
 * parameter, then (adam_m and adam_v given) one Adam step (Kingma and Ba,
 * Algorithm 1, bias-corrected with step t):
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   p -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
 * rays_o, rays_d, target_rgb: device [n_rays, 3]; t_near, t_far: device
 * [n_rays]; params, adam_m, adam_v: device float32 [nerf_train_param_count]
 * (updated in place; params is read before it is updated); grad: optional
 * device float32 [nerf_train_param_count], the gradient before the update;
 * loss: device float32 [1]; rgb: optional device [n_rays, 3], the rendered
 * colours.  Weight gradients are sums over samples in a fixed order: a
 * step is deterministic.  workspace: device, 256-byte aligned, at least
 * nerf_train_workspace_size bytes, or NULL (allocated stream-ordered and
 * freed after the work).  The page's two-network step (coarse and fine
 * networks, MSE of both renderings) is two calls: the coarse network on
 * stratified samples with cfg.weights set, nerf_sample_pdf on those weights
 * (z_merged), then the fine network with cfg.z = z_merged; the sampled
 * depths carry no gradient, so each network's gradient is that of its own
 * term.  Errors: null pointers, unsupported network, n_samples outside
 * 1..256, n_rays * n_samples above 2^28, step < 1 with Adam, one of
 * adam_m/adam_v missing, misaligned z or weights, workspace too small. */
nerf_status nerf_train_step(const float* rays_o, const float* rays_d, const float* t_near, const float* t_far,
                            const float* target_rgb, int64_t n_rays, const nerf_train_cfg* cfg, float* params,
                            float* adam_m, float* adam_v, int64_t step, float* grad, float* loss, float* rgb,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Decoder of the hash-grid INR ("Instant-NGP - Visual Experiments", shared
 * toolkit HashINR): Linear(2L -> hidden), ReLU, Linear(hidden -> n_out) on
 * the concatenated grid features. */
typedef struct {
    int32_t hidden;        /* 1..64 */
    int32_t n_out;         /* 1..4 */
    float lr, beta1, beta2, eps; /* Adam */
} nerf_hash_inr_cfg;

/* Flat parameter count of the hash-grid INR on grid g: 2 floats per table
 * entry (levels back to back, as g's offsets), then W1 [hidden][2L], b1
 * [hidden], W2 [n_out][hidden], b2 [n_out] (0 if g or cfg is invalid). */
int64_t nerf_hash_inr_param_count(const nerf_hashgrid* g, const nerf_hash_inr_cfg* cfg);

/* Device workspace of nerf_hash_inr_train_step for n points (0 if invalid). */
size_t nerf_hash_inr_workspace_size(const nerf_hashgrid* g, const nerf_hash_inr_cfg* cfg, int64_t n);

/* One full-batch training step of the hash-grid INR ("Instant-NGP - Visual
 * Experiments (a 2D multiresolution hash grid)", shared toolkit HashGrid2D,
 * HashINR and train; Experiment 2): the grid features of each point (as
 * nerf_encode_hashgrid, but from learnable float32 tables inside params and
 * times g->level_mask), the decoder, loss = mean over points and outputs of
 * (prediction - target)^2, the gradient of every table entry and decoder
 * parameter (a point's feature gradient reaches each of its corners' entries
 * times the corner's weight and the level's mask), then (adam_m and adam_v
 * given) one bias-corrected Adam step as in nerf_train_step.  g: host grid
 * layout (dim 2 or 3, at most 16 levels; g->tables is not used).  x: device
 * [n, dim] in [0,1]^dim, 16-byte aligned; target: device [n, n_out];
 * params (16-byte aligned), adam_m, adam_v: device float32
 * [nerf_hash_inr_param_count] (params updated in place);
 * grad: optional device [nerf_hash_inr_param_count], the gradient before the
 * update; loss: device float32 [1]; pred: optional device [n, n_out].  The
 * decoder gradients and the loss are summed in a fixed order.  Table
 * gradients of levels with at most 32768 entries are exact integer sums of
 * per-thread float32 partial sums (consecutive points, in order) rounded to
 * 2^-32 in units of the output residual (each such partial clamped to
 * +-2048), so the step is deterministic; larger levels add up with float
 * atomics, whose last bits depend on the order in which points arrive.  workspace: device, 256-byte
 * aligned, at least nerf_hash_inr_workspace_size bytes (about 8 L bytes per
 * point, plus partial sums), or NULL (allocated stream-ordered).  Errors:
 * null pointers, bad grid layout or cfg, n above 2^27, step < 1 with Adam,
 * one Adam moment missing, workspace too small. */
nerf_status nerf_hash_inr_train_step(const float* x, const float* target, int64_t n, const nerf_hashgrid* g,
                                     const nerf_hash_inr_cfg* cfg, float* params, float* adam_m, float* adam_v,
                                     int64_t step, float* grad, float* loss, float* pred, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* For callers that cannot allocate                                       */
/* ---------------------------------------------------------------------- */

/* Bytes of the fixed device scratch of nerf_render_noalloc (per device). */
#define NERF_NOALLOC_SCRATCH_MB 128

/* nerf_render for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * same arguments, results and validation as nerf_render, but no call to
 * hipMalloc/hipMallocAsync/hipFree or any allocating routine.  The
 * many-network mode (the only one with a workspace) takes its workspace from
 * a fixed array of NERF_NOALLOC_SCRATCH_MB MiB that the library holds on
 * each device from load to process end; cfg.workspace must be NULL, and the
 * rays are rendered in the largest chunks whose workspace fits (cfg.chunk,
 * if set, must fit, else NERF_ERR_WORKSPACE with the sizes in
 * nerf_last_error()).  Every call on one device shares that device's array:
 * calls that overlap on one device (other streams, other threads) race and
 * must be serialised by the caller.  Results equal nerf_render's bit for bit
 * (they do not depend on the chunking). */
nerf_status nerf_render_noalloc(const float* rays_o, const float* rays_d, const float* t_near, const float* t_far,
                                int64_t n_rays, const nerf_weights* w, const nerf_render_cfg* cfg, float* rgb,
                                float* depth, float* acc, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NERF_MI355X_H */
