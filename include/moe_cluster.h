/*
 * moe_cluster.h -- host routine that (re)builds the compressed experts of
 * one MoE FFN layer: online dual-similarity clustering of E experts into G
 * groups of K = E/G, then a shared group base plus a rank-r residual per
 * expert.  It runs every few training steps, off the forward path, on the
 * CPU (C++, no device memory); its outputs are what moe_create takes.
 *
 * Source: "Breaking the MoE LLM Trilemma: Dynamic Expert Clustering with
 * Structured Compression" (papernotes.org note on arXiv 2510.02345).
 *   Key design 1: each expert keeps vec(W_i) and an activation centroid
 *   mu_i <- (1 - beta) mu_i + beta xbar_i; S_param = cos(vec W_i, vec W_j),
 *   S_task = cos(mu_i, mu_j), S = alpha S_param + (1 - alpha) S_task; pairs
 *   below tau leave the neighbour graph; K-means++ on D = 1 - S gives G
 *   groups, evened out by greedily moving boundary experts; S_param rows
 *   are cached for m reclusterings unless the expert's weights moved by
 *   more than eps.
 *   Key design 2: W_base^g = mean of the group's experts; the residual
 *   A_i B_i^T is the rank-r truncated SVD of W_i - W_base^g (A_i d_in x r,
 *   B_i d_out x r), which keeps the Frobenius error small (1.5% at r = 16
 *   on the page's models).
 *
 * Where the page leaves a step open the routine takes these readings:
 *   xbar_i = mean of the rows routed to expert i in the observed batch (an
 *   expert with no row keeps mu_i; centroids start at zero); cos(0, v) = 0;
 *   vec(W_i) concatenates all projections; a pair below tau gets S = 0;
 *   the clustering is k-medoids with k-means++ seeding driven by caller
 *   uniforms u[G] (seed 0 = expert floor(u_0 E); seed j = first expert whose
 *   running sum of squared distances to the nearest seed exceeds u_j times
 *   the total), alternating nearest-medoid assignment (ties to the lower
 *   group) and medoid update (the member with the least distance sum, ties
 *   to the lower expert) until the medoids repeat; evening out moves, one at
 *   a time, the member of an over-full group whose move to an under-full
 *   group raises its medoid distance least (ties: lower expert, then lower
 *   group) until every group has K; the cache recomputes expert i when its
 *   age reaches m or ||W_i - W_i^cached|| > eps ||W_i^cached||; the
 *   singular values are split evenly, A = U_r sqrt(S_r), B = V_r sqrt(S_r);
 *   after regrouping expert j of group g (ascending expert order) is stored
 *   at index g*K + j.
 *
 * All functions return MOE_OK (0) or an error code from moe.h, with
 * moe_last_error() describing a failure.  Every pointer is a HOST pointer.
 * A moe_cluster object is not thread-safe.
 */
#ifndef CEFN_MOE_CLUSTER_H
#define CEFN_MOE_CLUSTER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t E;          /* experts */
  int32_t G;          /* groups; E % G == 0 */
  int32_t d;          /* token width (length of an activation centroid) */
  int64_t n_param;    /* length of vec(W_i) */
  double alpha;       /* weight of S_param in S (the page: above 0.5; 0.7 is ours) */
  double beta;        /* EMA rate of the centroids (the page: 0.05) */
  double tau;         /* neighbour-graph threshold (the page: 0.1) */
  double eps;         /* relative weight change that refreshes a cached S_param row */
  int32_t cache_life; /* m: reclusterings a cached row lives (>= 1) */
} moe_cluster_config;

typedef struct moe_cluster moe_cluster;

/* Create the clustering state (centroids zero, S_param cache empty). */
int moe_cluster_create(const moe_cluster_config* cfg, moe_cluster** out);
int moe_cluster_destroy(moe_cluster* c);

/* Read or replace the activation centroids, float64 [E][d]. */
int moe_cluster_get_centroids(const moe_cluster* c, double* mu);
int moe_cluster_set_centroids(moe_cluster* c, const double* mu);

/* One EMA step from a routed batch: X float32 [T][d], idx int32 [T][k]
 * (expert ids, distinct within a row; ids outside [0, E) are an error). */
int moe_cluster_observe(moe_cluster* c, const float* X, int32_t T, const int32_t* idx, int32_t k);

/* Regroup.  W[i] points to vec(W_i) (float32, n_param values) for every
 * expert i.  u: G uniforms in [0, 1) for the k-means++ seeding.  Writes
 * group_of [E] (the group of each expert) and members [G][K] (each group's
 * experts, ascending), and when non-NULL the fused, pruned similarity
 * S_out [E][E] and the list of experts whose S_param row was recomputed
 * (fresh [E]: 1 = recomputed, 0 = cached). */
int moe_cluster_regroup(moe_cluster* c, const float* const* W, const double* u, int32_t* group_of,
                        int32_t* members, double* S_out, int32_t* fresh);

/* Compress one projection for a grouping: W[i] points to expert i's dense
 * weights, float32 [d_in][d_out] row-major.  members [G][K] as written by
 * moe_cluster_regroup.  Writes base [G][d_in][d_out], A [E][d_in][r] and
 * B [E][d_out][r] (float32, expert j of group g at index g*K + j), and
 * when non-NULL rel_err [E], ||W_i - W~_i||_F / ||W_i||_F in float64 for the
 * stored float32 factors.  The truncated SVD is a block subspace iteration
 * in float64 (block r + 8, run until the rank-r subspace settles, at most
 * 200 rounds).  Threads: up to n_threads (0 = hardware concurrency). */
int moe_compress_projection(int32_t E, int32_t G, const int32_t* members, int32_t d_in, int32_t d_out,
                            int32_t r, const float* const* W, float* base, float* A, float* B,
                            double* rel_err, int32_t n_threads);

#ifdef __cplusplus
}
#endif
#endif /* CEFN_MOE_CLUSTER_H */
