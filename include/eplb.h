/*
 * eplb.h -- C ABI of the EPLB hot path on AMD Instinct MI355X (gfx950).
 *
 * Three calls make up the path: a per-layer expert-load histogram of top-k
 * routing ids summed over a window of steps, the batched rebalance that turns
 * loads into a replica placement (phy2log / log2phy / logcnt), and the
 * redirect of routed logical ids to physical replicas.  Around them: the
 * histogram and redirect fused in one pass, a moving-average load estimate,
 * the per-rank load of a placement (its max / mean), the plan of weight
 * copies that turns one placement into the next, and an LPLB-style
 * per-batch redistribution of tokens over replica edges.
 *
 * What each call computes is defined by the EPLB README and its annotated
 * source on the translation page «DualPipe и EPLB: конвейер в обе стороны и
 * балансировщик экспертов» (ai.flicky.cc), Part 2 "EPLB"; every declaration
 * below names the section it follows.
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers to contiguous, row-major memory
 *     that the caller allocates, owns and keeps alive until the work enqueued
 *     on `stream` has finished.  The library allocates, frees and synchronises
 *     nothing and keeps no state between calls.  The one call that needs
 *     working memory, eplb_lp_redirect, takes it as an argument; its variant
 *     eplb_lp_redirect_noalloc uses a fixed array of the library on each GPU
 *     instead.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; the return code reports host-side validation and launch
 *     only.  Calls on different streams may run concurrently provided their
 *     output buffers do not overlap.
 *   - A non-zero return code means nothing was enqueued (EPLB_E_HIP: a launch
 *     failed and earlier kernels of the same call may have run).
 *   - No output (in/out buffers such as `ring` and `ema` included) may share
 *     a byte with an input or with another output of the same call; the
 *     check compares address ranges and returns EPLB_E_ARG.
 *   - One call takes at most 2^22 layers (streaming calls) or 2^22 problems
 *     (rebalance-like calls), else EPLB_E_LIMIT, so that each launch stays
 *     below 2^32 work-items.
 *   - Conditions only the device can see are reported through output
 *     arguments (`n_invalid`, `status`), never by faulting.
 */
#ifndef EPLB_H_
#define EPLB_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes (host side) ------------------------------------------ */
#define EPLB_OK            0  /* enqueued                                          */
#define EPLB_E_ARG         1  /* NULL pointer or a size out of its range           */
#define EPLB_E_DIV         2  /* a divisibility rule of the placement is broken    */
#define EPLB_E_REDUNDANCY  3  /* fewer physical than logical experts (P < E)       */
#define EPLB_E_CAPACITY    4  /* log2phy width X below 1 + (P - E) / nodes         */
#define EPLB_E_LIMIT       5  /* problem larger than the kernels' on-chip budget   */
#define EPLB_E_RANGE       6  /* T * K >= 2^31 (ids per layer must fit int32)      */
#define EPLB_E_HIP         7  /* a HIP launch failed                               */

/* ---- per-problem status written by eplb_rebalance ------------------------ */
#define EPLB_S_OK          0  /* placement written                                 */
#define EPLB_S_BAD_LOAD   16  /* some load < 0 or > 2^40; outputs set to -1        */
#define EPLB_S_OVERFLOW   17  /* lcm(replica counts of a node) * (node load sum)
                                 >= 2^127; outputs set to -1                       */
#define EPLB_S_BAD_MAP    18  /* eplb_rearrange: an entry outside its range, or a
                                 new expert with no old replica; outputs -1        */
#define EPLB_S_BAD_TOPOLOGY 19 /* eplb_lp_solve: an id, home rank or count out of
                                 range, or an expert replicated twice; outputs -1  */

/*
 * eplb_load_hist -- expert load of one step, and the load over a window.
 *
 * Follows: the translator's glossary of Part 2 (the load of an expert is the
 * number of tokens the router sent to it in the observation period) and the
 * opening section of Part 2 (load is predicted from historical statistics,
 * e.g. a moving average).  The window here is a SUM of the last W per-step
 * histograms; the rebalance only compares loads, so a sum and an average
 * place experts identically.
 *
 *   idx        [L][T][K] int32   logical expert id of each (layer, token, k)
 *   L, T, K                      layers, tokens, top-k (0 <= L <= 2^22,
 *                                T >= 0, K >= 1, T * K < 2^31)
 *   E                            logical experts per layer (1 .. 4096)
 *   ring       [W][L][E] int32   caller-owned history of per-step counts.
 *                                Zero it once before the first step; this
 *                                call overwrites slot (step % W) with the
 *                                counts of `idx` and leaves the other slots.
 *   W, step                      window length (>= 1) and step number (>= 0)
 *   load       [L][E] int64      out: sum over all W slots of `ring`
 *   n_invalid  [L] int64         out: ids of layer l outside [0, E); they are
 *                                not counted
 *
 * Errors: EPLB_E_ARG (L or T < 0, K, E or W < 1, step < 0, a NULL array, or
 * ring, load or n_invalid sharing a byte with idx or with each other),
 * EPLB_E_LIMIT (E > 4096, L > 2^22), EPLB_E_RANGE (T * K >= 2^31),
 * EPLB_E_HIP.
 */
int32_t eplb_load_hist(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                       int32_t* ring, int32_t W, int64_t step,
                       int64_t* load, int64_t* n_invalid, void* stream);

/*
 * eplb_rebalance -- replica placement for B independent problems.
 *
 * Follows: Part 2 sections "Алгоритм" (hierarchical policy when the number
 * of nodes divides the number of groups, global policy otherwise), the
 * flowchart (the global policy is the same routine with one group on one
 * node), "Интерфейс и пример" (inputs and the meaning of phy2log), and the
 * appendix's packing, replication and three-step hierarchical routines.
 *
 *   load       [B][E] int64      token count per logical expert, 0 .. 2^40
 *   B                            problems (layers or load snapshots), >= 0
 *   E, P                         logical and physical experts per problem
 *   G, N, RK                     expert groups, nodes, ranks (GPUs)
 *   X                            width of log2phy, >= 1 + (P - E) / N'
 *                                where N' = N if G % N == 0 else 1
 *   phy2log    [B][P] int32      out: logical expert held by physical slot
 *                                p = node*(P/N') + gpu_in_node*(P/RK) + pos
 *   log2phy    [B][E][X] int32   out: physical slot of replica r of expert e
 *                                (r = 0 is the original), -1 for r >= logcnt
 *   logcnt     [B][E] int32      out: replicas of each logical expert (>= 1)
 *   status     [B] int32         out: EPLB_S_* per problem
 *
 * Exact, integer-only semantics (the pages use float32): loads per replica
 * are compared as exact rationals; sorts are stable (equal values keep
 * ascending index); ties between packs go to the lowest pack index; a tie in
 * load per replica goes to the lowest node-local expert index; one item per
 * pack is the identity assignment.
 *
 * Errors: EPLB_E_ARG (a size < 1, B < 0, a NULL array, or an output sharing
 * a byte with the input or another output), EPLB_E_DIV
 * (E % G on the hierarchical path, RK % N', P % RK), EPLB_E_REDUNDANCY
 * (P < E), EPLB_E_CAPACITY (X too small), EPLB_E_LIMIT (B > 2^22, E > 4096,
 * P > 8192, X > 65535, more than 512 experts or 512 GPUs on one node (the
 * global policy counts all of them as one node), more than 512 nodes, a
 * possible replica count above 16128, or a working set above 160 KiB of
 * LDS, the LDS of one gfx950 compute unit), EPLB_E_HIP.
 */
int32_t eplb_rebalance(const int64_t* load, int64_t B, int32_t E, int32_t P,
                       int32_t G, int32_t N, int32_t RK, int32_t X,
                       int32_t* phy2log, int32_t* log2phy, int32_t* logcnt,
                       int32_t* status, void* stream);

/*
 * eplb_redirect -- route every (token, k) to a physical replica.
 *
 * Follows: the glossary of Part 2 (an expert with two copies gives each about
 * half of its tokens).  Replica r = t mod logcnt[l][e] of expert
 * e = idx[l][t][k] serves token row t:
 *     out[l][t][k] = log2phy[l][e][t mod logcnt[l][e]]
 * An id outside [0, E), or a count outside [1, X], gives -1.
 *
 *   idx        [L][T][K] int32   logical ids (as for eplb_load_hist)
 *   log2phy    [L][E][X] int32   from eplb_rebalance
 *   logcnt     [L][E] int32      from eplb_rebalance
 *   out        [L][T][K] int32   out: physical ids; must not share a byte
 *                                with idx, log2phy or logcnt
 */
int32_t eplb_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                      const int32_t* log2phy, const int32_t* logcnt, int32_t X,
                      int32_t* out, void* stream);

/*
 * eplb_hist_redirect -- eplb_load_hist and eplb_redirect in one pass over idx.
 *
 * Follows the same passages as the two calls it combines.  Counts the step's
 * ids into ring slot (step % W), sums the window into `load`, and writes the
 * physical id of every (token, k) under the placement (log2phy, logcnt) given,
 * typically the one computed from the window before this step.  Every output
 * is identical to calling eplb_load_hist then eplb_redirect with the same
 * arguments; each id is read once instead of twice.  Arguments, layouts,
 * errors: as for those two calls (no output, ring included, may share a byte
 * with idx, log2phy, logcnt or another output).
 */
int32_t eplb_hist_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                           int32_t* ring, int32_t W, int64_t step, int64_t* load, int64_t* n_invalid,
                           const int32_t* log2phy, const int32_t* logcnt, int32_t X, int32_t* out,
                           void* stream);

/*
 * eplb_load_ema -- expert load of one step, and an integer moving average.
 *
 * Follows: the opening section of Part 2 (load is predicted from historical
 * statistics, a moving average being the usual way) and the glossary (load =
 * tokens routed to the expert).  An alternative to the window of
 * eplb_load_hist that keeps one int64 per expert instead of W histograms:
 *     ema[l][e] <- ema[l][e] - floor(ema[l][e] / 2^shift) + count[l][e]
 * a decay of 1 - 2^-shift per step in exact integer arithmetic.  From zero
 * with a steady count c it rises to [c * 2^shift, (c + 1) * 2^shift), so for
 * eplb_rebalance (loads <= 2^40) keep count * 2^shift below 2^40.
 *
 *   idx        [L][T][K] int32   logical ids (as for eplb_load_hist)
 *   count      [L][E] int32      out: this step's histogram
 *   shift                        0 .. 62 (0 keeps only the latest step)
 *   ema        [L][E] int64      in/out: the estimate; zero it once before
 *                                the first step; values must stay below 2^62
 *   n_invalid  [L] int64         out: ids of layer l outside [0, E)
 *
 * Errors: as for eplb_load_hist; EPLB_E_ARG also for shift outside 0 .. 62.
 */
int32_t eplb_load_ema(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E,
                      int32_t* count, int32_t shift, int64_t* ema, int64_t* n_invalid, void* stream);

/*
 * eplb_ema_redirect -- eplb_load_ema and eplb_redirect in one pass over idx.
 *
 * Follows the same passages as the two calls it combines.  Counts the step's
 * ids into `count`, folds them into `ema` (ema <- ema - (ema >> shift) +
 * count), and writes the physical id of every (token, k) under the placement
 * (log2phy, logcnt) given.  Every output is identical to calling
 * eplb_load_ema then eplb_redirect with the same arguments; each id is read
 * once instead of twice.  Arguments, layouts, errors: as for those two calls
 * (no output, ema included, may share a byte with idx, log2phy, logcnt or
 * another output).
 */
int32_t eplb_ema_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, int32_t* count,
                          int32_t shift, int64_t* ema, int64_t* n_invalid, const int32_t* log2phy,
                          const int32_t* logcnt, int32_t X, int32_t* out, void* stream);

/*
 * eplb_placement_load -- load of every rank under a placement, and max / mean.
 *
 * Follows: the glossary of Part 2 (each copy of an expert takes an equal
 * share of its tokens), the translator's hands-on exercise 2 after the
 * annotated source (sum weight / logcnt over the experts of each GPU and
 * compare max / mean between the policies) and the check of the worked
 * example under "Интерфейс и пример" (GPU loads 86.5 .. 156, mean 129).
 *     rank_load[b][r] = sum over s < P/RK of load[b][e] / logcnt[b][e],
 *                       e = phy2log[b][r * (P/RK) + s]
 *     imbalance[b]    = max_r rank_load[b][r] / (sum_e load[b][e] / RK),
 *                       1 when every load is 0
 * Works for any placement, also one computed from older loads (to decide
 * whether to rebalance).  Double precision: each rank load is within
 * (P/RK + 1) * 2^-53 relative of the exact rational, imbalance within
 * (P/RK + 3) * 2^-53.  logcnt is not checked against phy2log.
 *
 *   load       [B][E] int64      token counts, 0 .. 2^40
 *   phy2log    [B][P] int32      logical expert of each physical slot
 *   logcnt     [B][E] int32      replicas per logical expert
 *   B, E, P, RK                  problems (>= 0), logical experts, physical
 *                                experts, ranks (>= 1; RK divides P)
 *   rank_load  [B][RK] double    out
 *   imbalance  [B] double        out
 * A problem with a load outside [0, 2^40], a phy2log entry outside [0, E) or
 * a referenced count below 1 gets NaN in all its outputs.
 *
 * Errors: EPLB_E_ARG (a size out of range, a NULL array, or an output sharing
 * a byte with an input or the other output), EPLB_E_DIV (P % RK != 0),
 * EPLB_E_LIMIT (E > 4096, so that the int64 total of the loads, at most
 * E * 2^40, is exact as a double; B > 2^22), EPLB_E_HIP.
 */
int32_t eplb_placement_load(const int64_t* load, const int32_t* phy2log, const int32_t* logcnt,
                            int64_t B, int32_t E, int32_t P, int32_t RK,
                            double* rank_load, double* imbalance, void* stream);

/*
 * eplb_rearrange -- which expert weights to copy where when a new placement
 * replaces the one in force, keeping every replica that can stay.
 *
 * Follows: the pages stop at the placement (the rebalance assigns replicas
 * to GPUs: opening section and "Алгоритм" of Part 2) and say nothing of
 * moving weights; this is the plain completion.  The new placement stays
 * rank for rank and is permuted only within each rank (positions inside a
 * GPU are interchangeable):
 *   - rank r holds slots [r*ppr, (r+1)*ppr), ppr = P / RK;
 *   - for each expert e, the first m old slots of the rank holding e are
 *     kept, m = min(copies of e on the rank before, after), matched in order
 *     to the first m new slots holding e;
 *   - the other new slots of the rank, ascending, take the rank's other old
 *     slots, ascending;
 *   - a slot that changes copies its expert from an old slot holding it: on
 *     the same rank if there is one (always a kept slot), else on the same
 *     node (slot s is on node s / (P/N)), else anywhere; the lowest slot of
 *     that class.  Sources refer to the OLD placement: a copy out of a slot
 *     that also changes must read it before it is overwritten.
 * The number of copies, per rank ppr minus the overlap of the two multisets,
 * is the least any within-rank permutation of the new placement needs.
 *
 *   old_phy2log  [B][P] int32    the placement in force
 *   new_phy2log  [B][P] int32    the new placement (from eplb_rebalance)
 *   new_log2phy  [B][E][X] int32 its log2phy (-1 padded); entries are mapped
 *                                through the same permutation, replica
 *                                order kept (not checked against phy2log)
 *   B, E, P, RK, N, X            problems, logical experts, physical experts,
 *                                ranks, nodes (RK % N == 0), log2phy width
 *   phy2log      [B][P] int32    out: the new placement, permuted in ranks
 *   log2phy      [B][E][X] int32 out: its log2phy
 *   src          [B][P] int32    out: old slot to copy slot p from; -1 kept
 *   moves        [B][3] int32    out: copies from the same rank, the same
 *                                node, another node
 *   status       [B] int32       out: EPLB_S_OK or EPLB_S_BAD_MAP
 * No output may share a byte with an input or another output.
 *
 * Errors: EPLB_E_ARG (a size < 1, B < 0, a NULL array, an output sharing a
 * byte with an input or another output), EPLB_E_DIV (P % RK, RK % N),
 * EPLB_E_LIMIT (E > 4096, P > 8192, X > 65535, B > 2^22), EPLB_E_HIP.
 */
int32_t eplb_rearrange(const int32_t* old_phy2log, const int32_t* new_phy2log, const int32_t* new_log2phy,
                       int64_t B, int32_t E, int32_t P, int32_t RK, int32_t N, int32_t X,
                       int32_t* phy2log, int32_t* log2phy, int32_t* src, int32_t* moves, int32_t* status,
                       void* stream);

/*
 * eplb_lp_solve -- per-batch redistribution of tokens over a fixed replica
 * topology (LPLB-style), exact in integers.
 *
 * Follows: the two LPLB pages, «DeepSeek开源LPLB：基于线性规划的MoE负载均衡器…»
 * (2048ai.net; items 4, 5 and 7: replica topology, LP model, topologies) and
 * the Machine Heart report on LPLB (wwwcj777.com, «LPLB 的工作原理»): each
 * redundant expert is an edge from its original's rank to its own rank that
 * can carry up to the expert's tokens of the batch; tokens move along the
 * edges to even out the ranks.  The pages leave the program unwritten; here:
 *     minimise lam over integer flows 0 <= flow[g][j] <= cnt[rep[g][j]]
 *     subject to, for every rank r,
 *       base[r] - (flows of r's experts to other ranks) + (flows into r) <= lam
 * with base[r] = sum of cnt[e] over the experts e with home[e] == r.
 * lam is unique; the flows are the ones a shortest-augmenting-path maximum
 * flow (lowest-numbered predecessor at each level) finds at lam, with each
 * rank pair's net flow split over the pair's slots in ascending slot order.
 *
 *   cnt        [B][E] int64      tokens routed to each logical expert in the
 *                                batch, 0 .. 2^40
 *   home       [B][E] int32      rank holding each expert's original
 *   rep        [B][RK][R] int32  expert replicated in slot j of rank g, or -1;
 *                                an expert has at most one replica (a replica
 *                                on its own home rank carries nothing)
 *   B, E, RK, R                  problems, experts, ranks (1 .. 64), slots
 *                                per rank (1 .. 64)
 *   lam        [B] int64         out: the least reachable largest rank load
 *   flow       [B][RK][R] int64  out: tokens slot (g, j) takes from the
 *                                original of rep[g][j] (0 for empty slots)
 *   rank_load  [B][RK] int64     out: rank loads after the moves (max = lam)
 *   status     [B] int32         out: EPLB_S_OK or EPLB_S_BAD_TOPOLOGY
 * No output may share a byte with an input or another output (with 12 to
 * 16 ranks rank_load also carries partial results between the call's two
 * launches).
 *
 * Errors: EPLB_E_ARG (a size < 1, B < 0, a NULL array, an output sharing a
 * byte with an input or another output), EPLB_E_LIMIT (E > 4096, RK > 64,
 * R > 64, B > 2^20 - 1), EPLB_E_HIP.
 */
int32_t eplb_lp_solve(const int64_t* cnt, const int32_t* home, const int32_t* rep, int64_t B, int32_t E,
                      int32_t RK, int32_t R, int64_t* lam, int64_t* flow, int64_t* rank_load, int32_t* status,
                      void* stream);

/*
 * eplb_lp_redirect -- route every (token, k) by the flows of eplb_lp_solve.
 *
 * Follows: the LPLB usage example on «DeepSeek开源LPLB…» (the planner maps
 * the model's logical ids to physical ones; physical experts are the E
 * logical ones followed by RK * R redundant slots) and the flows above.  In
 * each layer the occurrences of expert x are numbered 0, 1, ... in (token, k)
 * order; if x has a replica in slot (g, j), the first flow[g][j] of them go
 * there, the rest to the original:
 *     out = E + g*R + j   for occurrence i < flow[g][j],   else   out = x
 * An id outside [0, E) gives -1; so does every id of a layer whose rep names
 * an id outside [0, E) or an expert twice.
 *
 *   idx        [L][T][K] int32   logical ids of the batch
 *   rep        [L][RK][R] int32  replica slots (as for eplb_lp_solve)
 *   flow       [L][RK][R] int64  tokens each slot takes (eplb_lp_solve)
 *   RK, R                        ranks (1 .. 64) and slots per rank (1 .. 64)
 *   workspace                    caller-owned device memory of at least
 *                                eplb_lp_redirect_workspace_bytes(L, T, K, E)
 *                                bytes (per-segment counts; contents on entry
 *                                do not matter and are overwritten)
 *   workspace_bytes              its size
 *   out        [L][T][K] int32   out: physical ids; must not share a byte
 *                                with idx, rep or flow
 *
 * Errors: as for eplb_redirect; EPLB_E_ARG also for RK or R < 1, a NULL
 * array or workspace, a workspace below the size needed, or a workspace
 * sharing a byte with idx, rep, flow or out; EPLB_E_LIMIT for RK > 64, R > 64, or more
 * than 2^25 segments of 2048 ids over all layers.
 */
int32_t eplb_lp_redirect(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, const int32_t* rep,
                         const int64_t* flow, int32_t RK, int32_t R, void* workspace, int64_t workspace_bytes,
                         int32_t* out, void* stream);

/* Bytes of workspace eplb_lp_redirect needs: L * ceil(T*K / 2048) * E * 4,
 * or a negative EPLB_E_* code.  Host only. */
int64_t eplb_lp_redirect_workspace_bytes(int64_t L, int64_t T, int32_t K, int32_t E);

/*
 * eplb_lp_redirect_noalloc -- eplb_lp_redirect for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It calls no allocating routine; its
 * per-segment counts live in a fixed array of the library on each GPU
 * (EPLB_NOALLOC_SCRATCH_BYTES, held until the process ends; its address is
 * looked up on the first call on each device).
 *
 * Arguments, layouts, outputs and errors: as for eplb_lp_redirect, without
 * the workspace; in addition EPLB_E_LIMIT when the counts need more than the
 * array holds, L * ceil(T*K / 2048) * min(E, RK * R) * 4 bytes >
 * EPLB_NOALLOC_SCRATCH_BYTES (for example 58 layers of 16384 tokens x top-8
 * with 64 replica slots need 950,272 bytes), and EPLB_E_HIP if the array's
 * address cannot be found.  All calls on one GPU share the array: calls that
 * overlap in time on one GPU (different streams or threads) race; calls on
 * one stream are ordered and safe.  Nothing in the array needs clearing.
 */
#define EPLB_NOALLOC_SCRATCH_BYTES (4 * 1024 * 1024)
int32_t eplb_lp_redirect_noalloc(const int32_t* idx, int64_t L, int64_t T, int32_t K, int32_t E, const int32_t* rep,
                                 const int64_t* flow, int32_t RK, int32_t R, int32_t* out, void* stream);

/*
 * eplb_rebalance_max_count -- the largest replica count eplb_rebalance can
 * give one logical expert, 1 + (P - E) / N' (N' = N if G % N == 0 else 1),
 * which is the least log2phy width X it accepts, or a negative EPLB_E_*
 * code (-EPLB_E_ARG for a size < 1, -EPLB_E_DIV for E % G on the
 * hierarchical path, -EPLB_E_REDUNDANCY for P < E).  Host only.
 *
 * Follows: the appendix entry point of Part 2 (log2phy is as wide as the
 * largest count) and the replication routine (a node adds (P - E) / N'
 * replicas, at most all of them to one expert).
 */
int32_t eplb_rebalance_max_count(int32_t E, int32_t P, int32_t G, int32_t N);

/* Human-readable name of an EPLB_E_* return code or EPLB_S_* status. */
const char* eplb_status_string(int32_t code);

/*
 * eplb_rebalance_lds_bytes -- the LDS working set of one rebalance problem,
 * in bytes, or a negative EPLB_E_* code if the arguments are invalid.  Host
 * only; touches no device.  Lets a caller check EPLB_E_LIMIT ahead of time.
 */
int64_t eplb_rebalance_lds_bytes(int32_t E, int32_t P, int32_t G, int32_t N,
                                 int32_t RK, int32_t X);

#ifdef __cplusplus
}
#endif

#endif /* EPLB_H_ */
