"""Write the hand-derived closed-form fixtures in this folder.

The expected values are the attention gradient worked out by hand for inputs
chosen so that the softmax has simple rational probabilities (each step is in
the `derivation` field).  No library and no oracle code is involved: only
`math.log` to print ln 3 and ln 4.  Run: python tests/golden/make_closed_forms.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ln3 = math.log(3.0)

ONE_QUERY_TWO_KEYS = {
    "citation": "Attention gradient in closed form.  Method equations: sm90 backward "
                "page, mma_one_m_block (scores, P = exp(S - LSE), dP = dO V^T, "
                "dS = P (dP - rowsum), dV = P^T dO, dQ = dS K, dK = dS^T Q); softmax "
                "scale on dQ and dK as on the Triton FA2 teaching page (dQ kernel).",
    "derivation": [
        "S = scale*q*k = [0, ln 3]; LSE = ln(1+3) = ln 4; P = [1/4, 3/4]; O = 3/4*4 = 3",
        "dP = dO*v = [0, 4]; sum_k P_k dP_k = 3; dS = P*(dP-3) = [-3/4, 3/4]",
        "dQ = scale*sum_j dS_j k_j = (3/4) ln 3; dK_j = scale*dS_j*q = [-3/4, 3/4]; "
        "dV_j = P_j*dO = [1/4, 3/4]"],
    "shape": {"H": 1, "Hk": 1, "Sq": 1, "Sk": 2, "D": 1}, "scale": 1.0, "causal": False,
    "q": [[[1.0]]], "k": [[[0.0]], [[ln3]]], "v": [[[0.0]], [[4.0]]], "dout": [[[1.0]]],
    "out": [[[3.0]]], "lse": [[math.log(4.0)]],
    "dq": [[[0.75 * ln3]]], "dk": [[[-0.75]], [[0.75]]], "dv": [[[0.25]], [[0.75]]],
}

CAUSAL_BOTTOM_RIGHT_2X3 = {
    "citation": "Closed form with the bottom-right causal rule of the GQA/MQA page "
                "(causal block bound: key limit of row i is i + seqlen_k - seqlen_q) "
                "and the method equations of the sm90 backward page, mma_one_m_block.",
    "derivation": [
        "Sq=2, Sk=3, causal bottom-right: row 0 sees keys 0,1; row 1 sees keys 0,1,2",
        "row 0: S = 0.5*2*k = [0, ln 3, masked]; P = [1/4, 3/4, 0]; O = 3; LSE = ln 4",
        "row 1: q = 0 so S = [0,0,0]; P = [1/3,1/3,1/3]; O = 5/3; LSE = ln 3",
        "row 0: dP = 1*v = [0,4,1]; rowsum = 3; dS = [-3/4, 3/4, 0]",
        "row 1: dP = 3*v = [0,12,3]; rowsum = 5; dS = [-5/3, 7/3, -2/3]",
        "dQ0 = 0.5*(3/4 ln 3) = (3/8) ln 3; dQ1 = 0.5*((7/3) ln 3 - (2/3)*5) "
        "= (7/6) ln 3 - 5/3",
        "dK_j = 0.5*(2*dS0j + 0*dS1j) = [-3/4, 3/4, 0]",
        "dV_j = P0j*1 + P1j*3 = [5/4, 7/4, 1]"],
    "shape": {"H": 1, "Hk": 1, "Sq": 2, "Sk": 3, "D": 1}, "scale": 0.5, "causal": True,
    "q": [[[2.0]], [[0.0]]], "k": [[[0.0]], [[ln3]], [[5.0]]],
    "v": [[[0.0]], [[4.0]], [[1.0]]], "dout": [[[1.0]], [[3.0]]],
    "out": [[[3.0]], [[5.0 / 3.0]]], "lse": [[math.log(4.0)], [math.log(3.0)]],
    "dq": [[[0.375 * ln3]], [[7.0 / 6.0 * ln3 - 5.0 / 3.0]]],
    "dk": [[[-0.75]], [[0.75]], [[0.0]]], "dv": [[[1.25]], [[1.75]], [[1.0]]],
}

SOFTCAP_ONE_QUERY_TWO_KEYS = {
    "citation": "Closed form with soft-capped scores: the softcap argument of mha_bwd on "
                "the backward call-trace page, read as c * tanh(x / c) of the scaled score "
                "x, and the method equations of the sm90 backward page, mma_one_m_block; "
                "the gradient passes the cap by the chain rule.",
    "derivation": [
        "c = 2 ln 3, scale = 1/2, q = 2: x = scale*q*k = k = [0, (ln 3)^2]",
        "x / c = [0, (ln 3)/2] and tanh((ln 3)/2) = (3-1)/(3+1) = 1/2, so the capped "
        "scores are c*[0, 1/2] = [0, ln 3]",
        "P = [1/4, 3/4]; O = 3/4*4 = 3; LSE = ln 4",
        "dS with respect to the capped scores (as without a cap): [-3/4, 3/4]",
        "cap derivative 1 - tanh^2 = [1, 3/4]; dS with respect to x: [-3/4, 9/16]",
        "dQ = scale*sum_j dS_j k_j = (1/2)(9/16)(ln 3)^2 = (9/32)(ln 3)^2; "
        "dK_j = scale*dS_j*q = [-3/4, 9/16]; dV_j = P_j*dO = [1/4, 3/4]"],
    "shape": {"H": 1, "Hk": 1, "Sq": 1, "Sk": 2, "D": 1}, "scale": 0.5, "causal": False,
    "softcap": 2.0 * ln3,
    "q": [[[2.0]]], "k": [[[0.0]], [[ln3 * ln3]]], "v": [[[0.0]], [[4.0]]],
    "dout": [[[1.0]]], "out": [[[3.0]]], "lse": [[math.log(4.0)]],
    "dq": [[[9.0 / 32.0 * ln3 * ln3]]], "dk": [[[-0.75]], [[9.0 / 16.0]]],
    "dv": [[[0.25]], [[0.75]]],
}

if __name__ == "__main__":
    for name, obj in (("closed_form_one_query_two_keys.json", ONE_QUERY_TWO_KEYS),
                      ("closed_form_causal_bottom_right_2x3.json", CAUSAL_BOTTOM_RIGHT_2X3),
                      ("closed_form_softcap_one_query_two_keys.json",
                       SOFTCAP_ONE_QUERY_TWO_KEYS)):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(obj, f, indent=1)
    print("written")
