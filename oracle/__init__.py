"""CPU oracle for the block-sparse spatiotemporal attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  It is plain numpy in
float64, shares no code with the HIP library, and is written from the method
descriptions on the five pages:

* "[논문리뷰] LVSA: Training-Free Sparse Attention for Long Video Diffusion"
  (blog review), section 1 Key Terms and section 3 Method & Key Results:
  block-sparse attention where each frame attends to a local window of frames
  and to global anchor frames whose positions rotate at every denoising step.
* "라디얼 어텐션, 비디오 확산 모델에서 비용 4.4배 절감하며 품질 유지" (hyper.ai
  headline on Radial Attention): a static mask whose attention window shrinks
  exponentially with temporal distance, O(n log n).
* "SVG-EAR: Parameter-Free Linear Compensation for Sparse Video Generation via
  Error-aware Routing", technical summary section 2 Method: centroid linear
  compensation of skipped blocks, error estimation with query-cluster
  centroids as proxies, error-to-cost routing under a density budget.
* "LinVideo: A Post-Training Framework towards O(n) Attention in Efficient
  Video Generation", technical summary sections 1-2: O(n) linear attention,
  and section 2 A: the mixed (r-weighted) form.
* "LIPAR: 비디오 생성 AI 를 위한 '스마트 스킵' 기술" (gist.science summary),
  section 2 B: latent inter-frame pruning and restoration.

Modules: ``mask`` (block rule and CSR), ``attention`` (block-sparse softmax
attention), ``svg_ear`` (centroids, routing scores, budget selection,
compensated attention; the score is pinned to the page's statement that the
estimated error converges to the actual error, see that module), ``linear`` (elu+1 linear attention, causal and
mixed forms), ``lipar`` (pruning and restoration), ``kmeans`` (the token
clustering and cluster order in front of the SVG-EAR calls),
``attention_bwd`` (gradients of the block-sparse attention).
"""

from . import mask, attention, attention_bwd, linear, svg_ear, lipar, kmeans  # noqa: F401
