"""TEST INFRASTRUCTURE ONLY: the plain CPU oracle (see ``oracle.py``).  Never imported by the product
package ``mlp_neural_shading_amd``."""
