// Affinity-aware sharding for delayed tensor parallelism (sptl_affinity.cpp).  Internal to
// libsptl.so; the C ABI entry points validate the arguments.
#pragma once

#include <stdint.h>

namespace sptl {

// sum over heads h and neurons j placed on the same device of a[h * n_neurons + j]
double colocated_affinity(const double *a, int n_heads, int n_neurons, const int *head_dev, const int *neuron_dev);

// For a head layout, the neuron layout (n_neurons / tp per device) of largest co-located
// affinity (exact).
void balanced_neuron_assignment(const double *a, int n_heads, int n_neurons, int tp, const int *head_dev,
                                int *neuron_dev);

// Number of head layouts with n_heads / tp heads per device (saturates at 2^62).
int64_t head_layout_count(int n_heads, int tp);

// For a neuron layout, the head layout (n_heads / tp per device) of largest co-located affinity,
// by trying every one (the first best in lexicographic order).
void best_head_layout(const double *a, int n_heads, int n_neurons, int tp, const int *neuron_dev, int *head_dev);

// Coordinate ascent from the head layout in head_dev: each round assigns the neurons, then
// searches the head layouts; stops after a round that does not raise the score, or after
// max_rounds.  Leaves the last round's layouts and score; returns the rounds run.
int affinity_layout(const double *a, int n_heads, int n_neurons, int tp, int max_rounds, int *head_dev,
                    int *neuron_dev, double *score);

}  // namespace sptl
