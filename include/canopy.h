/*
 * canopy.h: C ABI of libcanopy, tree-structured speculative verification of one Gated
 * DeltaNet (gated delta-rule linear attention) layer on AMD Instinct MI355X (gfx950).
 *
 * The operation (the canopy project page, projects.dotslasha.me/p/canopy.md, "Science
 * background"): a draft tree of T tokens, numbered so that parents precede children, is
 * verified through one layer whose per-head state S is d_k x d_v = 128 x 128. Running the gated
 * delta rule (S~ = alpha S, u = beta (v - S~^T k), S = S~ + k u^T, o = S^T q) along every
 * node's root path from the committed state S0 gives every node's output o_i and pseudo-value
 * u_i. The library computes them without walking the tree: with l_i the log cumulative decay
 * over path(i) and Gamma_ij = exp(l_i - l_j), it builds the ancestor-masked, decay-weighted
 * matrices G (beta_i Gamma_ij k_i.k_j over strict ancestors) and C (Gamma_ij q_i.k_j over
 * path(i)), solves the unit lower-triangular system (I + G) U = R with
 * R_i = beta_i (v_i - exp(l_i) S0^T k_i), and reads out O = diag(exp l) Q S0 + C U
 * ("The tree closed form"). Commit rebuilds only the accepted path's state,
 * S_a = exp(l_a) S0 + sum_{j in path(a)} Gamma_aj k_j u_j^T ("What the commit kernel stores").
 *
 * Conventions for every call:
 *  - All array pointers are HIP device memory, C-contiguous, owned and allocated by the
 *    caller. The library keeps no pointer after a call returns and allocates nothing.
 *  - Calls only enqueue work on `stream` (0 = the null stream) and return; they do not
 *    synchronise. Inputs are read-only; outputs are fully overwritten.
 *  - d_k = d_v = 128. 1 <= T <= 256. B >= 1. Heads follow "Design decisions / Memory layout":
 *    q and k have H heads, v, alpha, beta, S0 and every per-head output have HV heads, and
 *    each q/k head serves HV / H value heads (grouped value heads, FLA's layout): value head j
 *    reads q/k head j / (HV / H). 1 <= H <= HV, H divides HV, B * HV * 256 <= INT_MAX. H = HV
 *    is the plain one-to-one layout.
 *  - Ragged batches ("Memory layout": the tree plus a per-sequence length): tree_len [B]
 *    int32 may be NULL (every tree has T nodes) or give sequence b's node count, 1..T. Arrays
 *    keep their T-row extent; the nodes past a sequence's length are padding: their inputs are
 *    never used (they may hold anything, NaN included) and their outputs are not written. A
 *    length outside 1..T is a malformed tree with status -1 (all T rows then count as the tree
 *    and hold NaN).
 *  - Node order is the caller's: node i's outputs sit at index i. parent[b,0] must be -1 and
 *    -1 <= parent[b,i] < i; further roots (parent -1) start from S0 too.
 *  - The scale on q is 1 (callers that want 1/sqrt(d_k) pre-scale q).
 *  - alpha must lie in (0, 1]; beta is any finite value (0 allowed).
 *  - q, k, v, S0, U, S_new, O (serial baseline) and snapshots must be 16-byte aligned.
 *  - Errors found on the host (null required pointer, misaligned array, bad size, dtype, solver
 *    or waves) return a status and launch nothing. A failed launch returns CANOPY_ERR_HIP. A malformed tree or
 *    path is found on the device without blocking: it is reported in tree_status/path_status
 *    and that sequence's outputs are NaN.
 */
#ifndef CANOPY_H
#define CANOPY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CANOPY_OK = 0,
    CANOPY_ERR_ARG = 1,         /* null required pointer or a size out of range */
    CANOPY_ERR_UNSUPPORTED = 2, /* dtype, solver or waves value not supported */
    CANOPY_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or smaller than required */
    CANOPY_ERR_HIP = 4          /* the HIP runtime reported a launch error */
} canopy_status;

typedef enum { CANOPY_FP32 = 0, CANOPY_BF16 = 1 } canopy_dtype;

/* How the unit lower-triangular system (I + G) U = R is solved ("Design decisions / Two solve
 * strategies"; "The tree closed form" for the Neumann series, its squaring form and the
 * level-synchronous solve). Three kernels serve the sizes:
 *  - T <= 16 (AUTO, NEUMANN): one wave per 16 value columns, all in registers; the Neumann
 *    series with one term per tree level.
 *  - 17 <= T <= 64 (AUTO, FWDSUB, NEUMANN): one wave per 16-node sub-block. FWDSUB and AUTO
 *    substitute forward over the sub-blocks, each 16 x 16 diagonal inverse formed as the
 *    squaring product (I + N)(I + N^2)(I + N^4)(I + N^8), N = -G_pp, truncated at the
 *    sub-block's depth; NEUMANN sums the whole tree's series, one term per tree level.
 *  - 65 <= T <= 256 with bf16 inputs (AUTO, FWDSUB), for at most 128 (sequence, head) pairs:
 *    the same wave-per-sub-block forward substitution, with the Gram tiles formed as the
 *    solved tiles arrive (16, 32 or 64 value columns per workgroup); the products of its
 *    sequential chain are bf16 hi + lo matrix-core passes (relative error about 2^-16).
 *  - 65 <= T <= 256 with bf16 inputs (AUTO, FWDSUB), for more than 256 pairs: 64-node blocks
 *    as below with FWDSUB on every diagonal block, in a kernel sized for two workgroups per CU
 *    (at most 80 KiB of LDS and 128 registers per lane: K_c rows, S0 and the solved U_c are
 *    read back from the caches instead of held), so that up to 512 pairs run in one pass. Its
 *    products are bf16 hi + lo matrix-core passes (relative error about 2^-16 per product).
 *  - Otherwise, and for LEVEL: 64-node blocks staged in LDS, the couplings to earlier blocks
 *    applied as matrix-core products; a diagonal block is solved by
 *      FWDSUB   forward substitution over four 16-node sub-blocks on fp32 matrix-core
 *               products, each 16 x 16 diagonal inverse formed as the truncated squaring
 *               product above;
 *      NEUMANN  the finite series sum_{m=0..d} (-G_bb)^m, d the block's in-block depth;
 *      LEVEL    row-by-row substitution with the rows of equal in-block depth together;
 *      AUTO     NEUMANN for blocks of in-block depth <= 2, FWDSUB otherwise (measured on
 *               level trees: the series wins at depth 0-2, substitution from 3 up).
 *  - LEVELSYNC (bf16 inputs, any T, one workgroup of 8 waves per (sequence, head)): the
 *    level-synchronous solve over the whole tree ("The tree closed form": level order, and the
 *    level-synchronous solve U_L = R_L - G_{L,:} U). Row i of G and C is non-zero only at the
 *    ancestors of i, so each node gathers over its own ancestor list: LDS tables hold one entry
 *    per (node, ancestor) pair, G and C of each pair formed on the matrix cores, and the u rows
 *    of the nodes that have a child. The nodes are taken in level order, 16 at a time (their
 *    K S0 and Q S0 rows on the matrix cores), every product of the solve and the read-out in
 *    fp32. Trees of at most 2560 (node, ancestor) pairs (sum of the node depths) and at most
 *    160 nodes with a child fit the tables; a larger tree runs the blocked solve with AUTO's
 *    choice for its blocks, so the result is the same system solved either way. Measured on
 *    MI355X at T = 256 it takes about as long per (sequence, head) as the blocked solve, so
 *    AUTO does not choose it.
 * Matrix-form solvers for any T (canopy_tree_verify_ws only: they keep T x T operators of each
 * (sequence, head) in a caller workspace). One launch per (sequence, head) builds N = -G and C
 * there; the solve then runs per (sequence, head, 16 value columns):
 *      SERIES   the whole tree's finite Neumann series (Bole's form): Z <- -G Z, U <- U + Z
 *               for d rounds, d the tree depth (G^(d+1) = 0);
 *      SQUARING the squaring form of the same series: Z <- (I + N^(2^k)) Z for
 *               k < ceil(log2(d + 1)), the powers squared once per (sequence, head);
 *      SPLIT    the split design ("Batch and heads to CTAs"): (I + G)^-1 multiplied out once per
 *               (sequence, head) as the squaring product, then applied per value tile. */
typedef enum {
    CANOPY_SOLVE_AUTO = 0,
    CANOPY_SOLVE_FWDSUB = 1,
    CANOPY_SOLVE_NEUMANN = 2,
    CANOPY_SOLVE_LEVEL = 3,
    CANOPY_SOLVE_SERIES = 4,
    CANOPY_SOLVE_SQUARING = 5,
    CANOPY_SOLVE_SPLIT = 6,
    CANOPY_SOLVE_LEVELSYNC = 7
} canopy_solver;

/* Library version, major * 10000 + minor * 100 + patch. */
int canopy_version(void);

/*
 * Test hook for failure handling (not part of the method). Some kernels hand results from one
 * wave to another inside a workgroup: the 17-64-node verify and the 65-256-node
 * wave-per-sub-block verify (solved sub-blocks of U), and canopy_hybrid_verify (fork
 * snapshots). A waiting wave sleeps between checks and gives up after `sleeps` sleeps; the
 * default, 2^24, is never reached (every publisher is resident and waits on nothing later).
 * A wave that gives up writes NaN for every output row it computes, passes the loss on to the
 * waves that wait for it in turn, and sets tree_status[b] = -2. Bound 0 makes every such wait
 * give up at once, so the whole path of a lost hand-off can be checked from the host with every
 * kernel still ending normally. sleeps < 0 restores the default. Applies to launches enqueued
 * after the call, in this process (one process-wide value); returns the previous bound.
 */
int canopy_set_wait_bound(int sleeps);

/* Text for a status code (static storage). */
const char *canopy_status_string(canopy_status s);

/*
 * Tree preprocessing on the GPU ("The tree closed form"; "Design decisions / Tree order and
 * tiling" for the T x T bitmask).
 *   parent      [B,T] int32, in.
 *   tree_len    [B] int32, in, may be NULL: per-sequence node counts (see above).
 *   alpha       [B,T,HV] fp32, in.
 *   anc_mask    [B,T,ceil(T/32)] uint32, out, may be NULL: bit (j % 32) of word j / 32 of row
 *               i is set iff j is in path(i) (strict ancestors and i itself).
 *   depth       [B,T] int32, out, may be NULL: |A(i)|, the root 0.
 *   ell         [B,T,HV] fp32, out, may be NULL: l_i = log alpha_i + l_parent(i), a root's
 *               parent counting 0, summed in fp64 and rounded once.
 *   tree_status [B] int32, out, may be NULL: 0; -1 for a tree_len outside 1..T; else 1 + the
 *               first node i whose parent is not in -1..i-1 (then mask and depth rows are 0
 *               and ell is NaN). The verify calls also report -2 when a wave gave up waiting
 *               for another wave's result (see canopy_set_wait_bound; the rows computed from it
 *               are NaN). The status of a valid tree is stored right after the tree
 *               preprocessing and a wait gives up only after its full bound, so -2 is the value
 *               left in place.
 */
canopy_status canopy_tree_prep(const int32_t *parent, const int32_t *tree_len, const float *alpha,
                               int B, int HV, int T, uint32_t *anc_mask, int32_t *depth, float *ell,
                               int32_t *tree_status, hipStream_t stream);

/*
 * Verify a draft tree through one GDN layer: every node's output and pseudo-value in one pass
 * (prep, S0 projections, masked Gram matrices, the triangular solve and the read-out fused).
 *   q, k        [B,T,H,128], in_dtype (fp32, or bf16 as 16-bit patterns), in.
 *   v           [B,T,HV,128], in_dtype, in.
 *   alpha, beta [B,T,HV] fp32, in.
 *   S0          [B,HV,128(k),128(v)] fp32, in: the committed state per (sequence, value head).
 *   parent      [B,T] int32, in.
 *   tree_len    [B] int32, in, may be NULL: per-sequence node counts.
 *   O, U        [B,T,HV,128] fp32, out: outputs o_i and pseudo-values u_i.
 *   ell         [B,T,HV] fp32, out: as in canopy_tree_prep.
 *   anc_mask, depth, tree_status: optional outputs (NULL to skip), as in canopy_tree_prep.
 *   solver      AUTO, FWDSUB, NEUMANN, LEVEL or LEVELSYNC (see canopy_solver; LEVELSYNC needs
 *               bf16 inputs and takes waves 0 or 8, else CANOPY_ERR_UNSUPPORTED); the matrix
 *               forms need a workspace and go through canopy_tree_verify_ws
 *               (CANOPY_ERR_UNSUPPORTED here).
 *   waves       workgroup width, 1, 2, 4, 8 or 16, or 0 to let the library choose from B, H
 *               and T.
 *               T <= 16 (AUTO, NEUMANN): 1, 2, 4 or 8 waves per workgroup, each owning 16
 *               value columns; 16 single-wave workgroups each owning 32 value columns (two
 *               16-column tiles). Waves 0 takes 16 with bf16 inputs when B*HV*8 single-tile
 *               waves would fill one pass of the GPU or more (3 per SIMD in
 *               canopy_commit_verify's one launch, 4 for the verify alone), else 1.
 *               17 <= T <= 64 (AUTO, FWDSUB, NEUMANN): 16-column tiles per workgroup, whose
 *               waves each own 16 nodes (8 is taken as 4).
 *               T > 64, bf16, AUTO or FWDSUB: 1 or 2 picks the wave-per-sub-block kernel with
 *               that many 16-column tiles per workgroup, 4 or 8 the blocked kernel, 16 the
 *               blocked kernel sized for two workgroups per CU (8 waves each; 16 needs bf16,
 *               T > 64, AUTO or FWDSUB and a head's rows of U and O within 2^31 bytes, else
 *               CANOPY_ERR_UNSUPPORTED).
 *               Otherwise (the blocked kernel): waves per workgroup, each owning 16 value
 *               columns; fp32 inputs use at most 2.
 */
canopy_status canopy_tree_verify(const void *q, const void *k, const void *v,
                                 const float *alpha, const float *beta, const float *S0,
                                 const int32_t *parent, const int32_t *tree_len, int B, int H,
                                 int HV, int T, canopy_dtype in_dtype, float *O, float *U,
                                 float *ell, uint32_t *anc_mask, int32_t *depth,
                                 int32_t *tree_status, canopy_solver solver, int waves,
                                 hipStream_t stream);

/*
 * Bytes of workspace canopy_tree_verify_ws needs for this batch and solver: 0 for the solvers
 * that need none (AUTO, FWDSUB, NEUMANN, LEVEL); for SERIES, SQUARING and SPLIT one slot per
 * (sequence, value head) of 64 + n * Tp * Tp * 4 bytes, Tp = T rounded up to 16, n = 3 (SERIES),
 * max(ceil(log2 T), 1) + 4 (SQUARING) or 11 (SPLIT). Returns 0 for sizes out of range.
 */
size_t canopy_workspace_bytes(int B, int HV, int T, canopy_solver solver);

/*
 * canopy_tree_verify with a caller workspace, for every solver including the matrix forms
 * (SERIES, SQUARING, SPLIT; see canopy_solver). Arguments and outputs as canopy_tree_verify,
 * plus:
 *   workspace        device memory of at least canopy_workspace_bytes(B, HV, T, solver) bytes,
 *                    16-byte aligned, owned by the caller; its contents are scratch (nothing
 *                    needs to be cleared before the call, nothing is kept after it). Calls that
 *                    share a workspace must not overlap in time. May be NULL when the solver
 *                    needs none.
 *   workspace_bytes  its size in bytes.
 *   waves            ignored by the matrix forms.
 * Errors: as canopy_tree_verify, plus CANOPY_ERR_WORKSPACE for a workspace that is NULL,
 * misaligned or too small when the solver needs one. The matrix forms take bf16 or fp32 inputs;
 * a malformed tree gives the status and NaN outputs as the other solvers do.
 */
canopy_status canopy_tree_verify_ws(const void *q, const void *k, const void *v,
                                    const float *alpha, const float *beta, const float *S0,
                                    const int32_t *parent, const int32_t *tree_len, int B, int H,
                                    int HV, int T, canopy_dtype in_dtype, float *O, float *U,
                                    float *ell, uint32_t *anc_mask, int32_t *depth,
                                    int32_t *tree_status, canopy_solver solver, int waves,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * canopy_tree_verify_ws for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels, with the
 * workspace taken from a device array inside the library (64 MiB per device, created with the
 * code object and held until the process ends) instead of a caller buffer. Allocates nothing.
 * Arguments, outputs and errors as canopy_tree_verify_ws without workspace and workspace_bytes;
 * a batch whose canopy_workspace_bytes exceeds 64 MiB returns CANOPY_ERR_WORKSPACE and launches
 * nothing (e.g. SPLIT at T = 256 fits 23 (sequence, head) pairs, SERIES at T = 256 fits 85).
 * Solvers that need no workspace go to canopy_tree_verify. Every call on a device shares that
 * device's array: calls on one device must not overlap in time (different streams included).
 */
canopy_status canopy_tree_verify_static(const void *q, const void *k, const void *v,
                                        const float *alpha, const float *beta, const float *S0,
                                        const int32_t *parent, const int32_t *tree_len, int B,
                                        int H, int HV, int T, canopy_dtype in_dtype, float *O,
                                        float *U, float *ell, uint32_t *anc_mask, int32_t *depth,
                                        int32_t *tree_status, canopy_solver solver, int waves,
                                        hipStream_t stream);

/*
 * Commit the accepted path: S_new = exp(l_a) S0 + sum_{j in path} exp(l_a - l_j) k_j u_j^T
 * with a the path's last node ("What the commit kernel stores"; "M5"). The decay ratios are
 * suffix sums of log alpha along the path (fp64), so no cancellation of large l enters them.
 *   S0          [B,HV,128,128] fp32, in.
 *   k           [B,T,H,128], in_dtype, in: the keys given to canopy_tree_verify.
 *   U           [B,T,HV,128] fp32, in: the pseudo-values canopy_tree_verify wrote.
 *   alpha       [B,T,HV] fp32, in.
 *   parent      [B,T] int32, in: only the path's own links are checked.
 *   tree_len    [B] int32, in, may be NULL: per-sequence node counts; path nodes must lie
 *               below them.
 *   path        [B,T] int32, in: node ids root first; entries past path_len are ignored.
 *   path_len    [B] int32, in: m in 0..n, n the sequence's node count (0 commits nothing:
 *               S_new = S0).
 *   S_new       [B,HV,128,128] fp32, out; may be the same memory as S0 (in place).
 *   path_status [B] int32, out, may be NULL: 0 valid, -1 path_len (or tree_len) out of range,
 *               else 1 + the first position t whose node is out of range or is not a child of
 *               path[t-1] (for t = 0: not a root). S_new of such a sequence is NaN.
 */
canopy_status canopy_commit(const float *S0, const void *k, canopy_dtype in_dtype,
                            const float *U, const float *alpha, const int32_t *parent,
                            const int32_t *tree_len, const int32_t *path, const int32_t *path_len,
                            int B, int H, int HV, int T, float *S_new, int32_t *path_status,
                            hipStream_t stream);

/*
 * One decode step of a layer: commit the previous tree's accepted path, then verify the new
 * draft tree from the committed state. The result equals canopy_commit followed by
 * canopy_tree_verify with S0 = S_new (the commit of "What the commit kernel stores" and the
 * closed form of "The tree closed form"; the two steps are only ordered, not changed). After a
 * previous tree of at most 64 nodes, both run in one launch and the committed state goes from
 * registers straight into the verify for new trees of at most 16 nodes (AUTO or NEUMANN) and
 * for 17 to 64 nodes (not LEVEL) when the 17-64 kernel's workgroups are narrow (B*HV <= 32, or
 * <= 128 at 49-64 nodes, with waves 0; or waves 1, or 2 at 49-64 nodes); otherwise the two
 * kernels run one after the other on the stream.
 *   S0, k_prev, U_prev, alpha_prev, parent_prev, tree_len_prev, path, path_len: as S0, k, U,
 *               alpha, parent, tree_len, path and path_len of canopy_commit, for the previous
 *               tree of T_prev nodes (k_prev [B,T_prev,H,128] in in_dtype).
 *   q, k, v, alpha, beta, parent, tree_len, solver, waves: as in canopy_tree_verify, for the
 *               new tree of T nodes.
 *   S_new       [B,HV,128,128] fp32, out: the committed state; may be the same memory as S0.
 *   path_status [B] int32, out, may be NULL: as in canopy_commit. A sequence whose path is
 *               rejected gets a NaN state, and its verify outputs are NaN as well.
 *   O, U, ell, anc_mask, depth, tree_status: as in canopy_tree_verify. With T == T_prev, U
 *               may be the same memory as U_prev (each value column of a head is read and
 *               written by the same wave, the reads first), so a decode loop of one tree
 *               size can keep one U buffer.
 * Errors: the checks of both calls, before anything is enqueued.
 */
canopy_status canopy_commit_verify(const float *S0, const void *k_prev, const float *U_prev,
                                   const float *alpha_prev, const int32_t *parent_prev,
                                   const int32_t *tree_len_prev, const int32_t *path,
                                   const int32_t *path_len, int T_prev, const void *q,
                                   const void *k, const void *v, const float *alpha,
                                   const float *beta, const int32_t *parent,
                                   const int32_t *tree_len, int B, int H, int HV, int T,
                                   canopy_dtype in_dtype, float *S_new, int32_t *path_status,
                                   float *O, float *U, float *ell, uint32_t *anc_mask,
                                   int32_t *depth, int32_t *tree_status, canopy_solver solver,
                                   int waves, hipStream_t stream);

/*
 * Every GDN layer's commit in one launch. After acceptance all L layers commit the same
 * accepted path on the same tree, each with its own state, keys, pseudo-values and gates, so
 * one launch serves them all (a decode step commits every layer at once). Arguments as
 * canopy_commit, with the per-layer ones given as HOST arrays of L device pointers
 * (1 <= L <= 64): S0[l], k[l], U[l], alpha[l], S_new[l] (S_new[l] may be S0[l]). path_status,
 * as in canopy_commit, is written once. Results equal L calls of canopy_commit bit for bit.
 */
canopy_status canopy_commit_layers(int L, const float *const *S0, const void *const *k,
                                   canopy_dtype in_dtype, const float *const *U,
                                   const float *const *alpha, const int32_t *parent,
                                   const int32_t *tree_len, const int32_t *path,
                                   const int32_t *path_len, int B, int H, int HV, int T,
                                   float *const *S_new, int32_t *path_status, hipStream_t stream);

/*
 * Serial fork baseline ("Design decisions / Serial baseline"): walk the nodes in order; each
 * node starts from its parent's per-node state snapshot (S0 for a root), takes one step of the
 * gated delta rule and writes its own snapshot, output and pseudo-value. Same inputs and
 * outputs as canopy_tree_verify plus
 *   snapshots   [B,T,HV,128,128] fp32, out: every node's state (padding nodes' not written).
 */
canopy_status canopy_serial_verify(const void *q, const void *k, const void *v,
                                   const float *alpha, const float *beta, const float *S0,
                                   const int32_t *parent, const int32_t *tree_len, int B, int H,
                                   int HV, int T, canopy_dtype in_dtype, float *O, float *U,
                                   float *snapshots, int32_t *tree_status, hipStream_t stream);

/*
 * Chain-decomposed hybrid ("What the papers report": SpecLA's chain-decomposed hybrid; "M4",
 * optional third contender): a heavy-light decomposition of the tree into chains, each chain
 * run serially with the state in registers, the chains in parallel, each starting as soon as
 * the snapshot it starts from is written. Same inputs and outputs as canopy_serial_verify,
 * except that only fork nodes (two or more children) get a snapshot: the other rows of
 * `snapshots` are not written. Its U feeds canopy_commit like canopy_tree_verify's.
 */
canopy_status canopy_hybrid_verify(const void *q, const void *k, const void *v,
                                   const float *alpha, const float *beta, const float *S0,
                                   const int32_t *parent, const int32_t *tree_len, int B, int H,
                                   int HV, int T, canopy_dtype in_dtype, float *O, float *U,
                                   float *snapshots, int32_t *tree_status, hipStream_t stream);

/*
 * Commit for the serial baseline: the accepted path's last node's snapshot (written by
 * canopy_serial_verify) becomes the new state (S0 itself for an empty path). Path checks and
 * path_status as in canopy_commit.
 *   snapshots   [B,T,HV,128,128] fp32, in.
 *   S0          [B,HV,128,128] fp32, in.
 *   S_new       [B,HV,128,128] fp32, out; may be the same memory as S0.
 */
canopy_status canopy_serial_commit(const float *snapshots, const float *S0, const int32_t *parent,
                                   const int32_t *tree_len, const int32_t *path,
                                   const int32_t *path_len, int B, int HV, int T, float *S_new,
                                   int32_t *path_status, hipStream_t stream);

/*
 * Root-path causal convolution of a draft tree (the canopy page, "M7", stretch item: the short
 * causal convolution before each GDN layer must follow each node's root path). Depthwise over
 * C channels with kernel size K:
 *   y_i[c] = sum_{j<K} w[c][j] * X_i(K-1-j)[c]   (then y = y * sigmoid(y) if silu = 1)
 * where X_i(0) = x_i, X_i(s) is the input s positions up node i's root path, and positions
 * before the root read the committed state, its last row first. Accumulates in fp32.
 *   x           [B,T,C], in_dtype (fp32, or bf16 as 16-bit patterns), in.
 *   w           [C,K] fp32, in: w[c][K-1] multiplies the node itself (a PyTorch depthwise
 *               conv1d weight [C,1,K] without its middle axis).
 *   conv_state  [B,K-1,C], in_dtype, in: the last K-1 committed inputs, oldest first.
 *   parent      [B,T] int32, in; tree_len [B] int32 or NULL, as for canopy_tree_verify.
 *   y           [B,T,C], in_dtype, out (bf16: rounded to nearest, ties to even); padding rows
 *               are not written; a malformed tree's rows are NaN.
 *   tree_status [B] int32, out, may be NULL: as in canopy_tree_prep.
 * 2 <= K <= 4, C a positive multiple of 8, 1 <= T <= 256. x, w, conv_state, y 16-byte aligned.
 */
canopy_status canopy_tree_conv(const void *x, canopy_dtype in_dtype, const float *w,
                               const void *conv_state, const int32_t *parent,
                               const int32_t *tree_len, int B, int T, int C, int K, int silu,
                               void *y, int32_t *tree_status, hipStream_t stream);

/*
 * Roll the convolution state forward over the accepted path ("commit must update the
 * convolution state with the accepted tokens"): state_new holds the last K-1 inputs of the
 * committed sequence (old state rows, then x of the path's nodes), oldest first. Path checks
 * and path_status as in canopy_commit; a bad sequence's state_new is NaN.
 *   x           [B,T,C], in_dtype, in: the inputs given to canopy_tree_conv.
 *   conv_state  [B,K-1,C], in_dtype, in.
 *   state_new   [B,K-1,C], in_dtype, out; may be the same memory as conv_state (in place).
 */
canopy_status canopy_conv_commit(const void *x, canopy_dtype in_dtype, const void *conv_state,
                                 const int32_t *parent, const int32_t *tree_len,
                                 const int32_t *path, const int32_t *path_len, int B, int T, int C,
                                 int K, void *state_new, int32_t *path_status, hipStream_t stream);

/*
 * canopy_serial_commit for L layers in one launch (host arrays of L device pointers,
 * 1 <= L <= 64; path_status written once), the serial baseline's counterpart of
 * canopy_commit_layers.
 */
canopy_status canopy_serial_commit_layers(int L, const float *const *snapshots,
                                          const float *const *S0, const int32_t *parent,
                                          const int32_t *tree_len, const int32_t *path,
                                          const int32_t *path_len, int B, int HV, int T,
                                          float *const *S_new, int32_t *path_status,
                                          hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CANOPY_H */
